"""The C ABI on the CPU: the library loads, exports every symbol the header
declares with the struct layout the binding uses, and rejects bad arguments
and bad metadata on the host (no device call is made on any of these paths).
"""
import ctypes
import os
import re
import subprocess

import pytest
import torch

from speculative_decode_amd import ops, workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
           if f.endswith(".h")]


def declared_functions():
    names = set()
    for h in HEADERS:
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^[A-Za-z_][\w\s\*]*?\b(gdn_\w+)\s*\(", text, flags=re.M):
            names.add(m.group(1))
    return names


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ops.LIB_PATH):
        import speculative_decode_amd.build as b
        b.build()
    return ops.load_library()


def test_library_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"gdn_spec_decode_update", "gdn_decode_update", "gdn_validate_indices_host",
            "gdn_last_error", "gdn_status_string"} <= names
    out = subprocess.run(["nm", "-D", "--defined-only", ops.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if l.strip()}
    assert names <= exported, names - exported
    assert names == set(ops.SIGNATURES), "binding and header disagree"


def test_abi_version_and_struct_layout(lib):
    assert lib.gdn_abi_version() == ops.ABI_VERSION
    hdr = open(os.path.join(ROOT, "include", "gdn_spec.h")).read()
    assert f"#define GDN_ABI_VERSION {ops.ABI_VERSION}" in hdr
    sizes = [ctypes.c_size_t() for _ in range(3)]
    lib.gdn_abi_struct_sizes(*[ctypes.byref(s) for s in sizes])
    assert [s.value for s in sizes] == [ctypes.sizeof(ops.GdnView), ctypes.sizeof(ops.GdnLayer),
                                        ctypes.sizeof(ops.GdnStatePool)]


def test_status_strings(lib):
    for code, name in ops.STATUS.items():
        assert lib.gdn_status_string(code).decode() == name


# -- argument checks: CPU tensors stand in for device buffers; the library only
#    reads their addresses and strides before it rejects the call ---------------
def _layer_and_pool(K=128, V=128, HK=1, HV=2, n_tok=4, act=torch.bfloat16, state=torch.bfloat16):
    q = torch.zeros(n_tok, HK, K, dtype=act)
    k = torch.zeros(n_tok, HK, K, dtype=act)
    v = torch.zeros(n_tok, HV, V, dtype=act)
    z = torch.zeros(n_tok, HV, V, dtype=act)
    a = torch.zeros(n_tok, HV, dtype=act)
    b = torch.zeros(n_tok, HV, dtype=act)
    out = torch.zeros(n_tok, HV, V, dtype=act)
    A_log = torch.zeros(HV)
    dt = torch.zeros(HV)
    w = torch.ones(V)
    pool = torch.zeros(4, HV, V, K, dtype=state)
    keep = (q, k, v, z, a, b, out, A_log, dt, w, pool)
    layer = ops.make_layer(q, k, v, z, a, b, A_log, dt, w, out)
    return layer, ops.make_pool(pool), keep


def _spec(lib, layer, pool, *, B=1, max_q_len=4, stride=4, meta=True):
    m = torch.zeros(16, dtype=torch.int32)
    p = ctypes.c_void_p(m.data_ptr()) if meta else None
    return lib.gdn_spec_decode_update(ctypes.byref(layer), ctypes.byref(pool), p, B, max_q_len,
                                      p, stride, p, None, None)


def test_valid_empty_batch_is_a_no_op(lib):
    layer, pool, keep = _layer_and_pool()
    assert _spec(lib, layer, pool, B=0) == 0
    m = torch.zeros(1, dtype=torch.int32)
    assert lib.gdn_decode_update(ctypes.byref(layer), ctypes.byref(pool),
                                 ctypes.c_void_p(m.data_ptr()), 0, None, None) == 0


@pytest.mark.parametrize("mutate,status,needle", [
    (lambda L, P: setattr(L, "head_k_dim", 64), 2, "head dims"),
    (lambda L, P: setattr(L, "head_v_dim", 256), 2, "head dims"),
    (lambda L, P: (setattr(L, "num_k_heads", 2), setattr(L, "num_v_heads", 3)), 1, "multiple"),
    (lambda L, P: setattr(L, "num_k_heads", 0), 1, "positive"),
    (lambda L, P: setattr(L, "act_dtype", 7), 2, "act_dtype"),
    (lambda L, P: setattr(L, "act_dtype", 3), 2, "act_dtype"),      # FP8 is a state format only
    (lambda L, P: setattr(L, "out_dtype", -1), 2, "out_dtype"),
    (lambda L, P: setattr(P, "dtype", 5), 2, "state dtype"),
    (lambda L, P: setattr(L.q, "data", None), 1, "q.data"),
    (lambda L, P: setattr(L.z, "data", L.z.data + 2), 1, "misaligned"),
    (lambda L, P: setattr(L.v, "stride_tok", 257), 1, "misaligned"),
    (lambda L, P: setattr(L.a, "stride_head", 2), 1, "stride_head"),
    (lambda L, P: setattr(L, "A_log", None), 1, "A_log"),
    # a float32 slice such as w[1:] is contiguous but only 4-byte aligned;
    # the kernels read norm_weight in pairs
    (lambda L, P: setattr(L, "norm_weight", L.norm_weight + 4), 1, "norm_weight must be 8-byte"),
    (lambda L, P: setattr(L, "norm_eps", -1.0), 1, "norm_eps"),
    (lambda L, P: setattr(P, "data", P.data + 8), 1, "16-byte"),
    (lambda L, P: setattr(P, "num_slots", 0), 1, "num_slots"),
])
def test_argument_errors(lib, mutate, status, needle):
    layer, pool, keep = _layer_and_pool()
    mutate(layer, pool)
    assert _spec(lib, layer, pool) == status
    assert needle in ops.last_error()
    assert lib.gdn_decode_update(ctypes.byref(layer), ctypes.byref(pool), None, 1, None,
                                 None) == status


def test_spec_entry_errors(lib):
    layer, pool, keep = _layer_and_pool()
    assert _spec(lib, layer, pool, max_q_len=9) == 2 and "exceeds" in ops.last_error()
    assert _spec(lib, layer, pool, max_q_len=0) == 1
    assert _spec(lib, layer, pool, stride=0) == 1
    assert _spec(lib, layer, pool, B=-1) == 1
    assert _spec(lib, layer, pool, meta=False) == 1 and "NULL" in ops.last_error()
    assert lib.gdn_spec_decode_update(None, ctypes.byref(pool), None, 1, 4, None, 4, None,
                                      None, None) == 1
    assert lib.gdn_decode_update(ctypes.byref(layer), ctypes.byref(pool), None, 2, None,
                                 None) == 1
    assert lib.gdn_decode_update(ctypes.byref(layer), ctypes.byref(pool), None, -2, None,
                                 None) == 1


def test_binding_checks_shapes_on_host():
    q = torch.zeros(4, 1, 128)
    with pytest.raises(ValueError):
        ops.make_layer(q, q, torch.zeros(4, 2, 128), torch.zeros(4, 2, 128),
                       torch.zeros(4, 3), torch.zeros(4, 2), torch.zeros(2), torch.zeros(2),
                       torch.ones(128), torch.zeros(4, 2, 128))
    with pytest.raises(ValueError):
        ops.make_pool(torch.zeros(2, 2, 128, 128).transpose(2, 3))


def test_binding_rejects_a_pool_that_does_not_match_the_layer(lib):
    """The kernels address tile (slot, h) as slot * HV + h with the layer's
    HV, so every entry point checks the pool's [HV, V, K] against the layer
    on the host, before anything is enqueued (CPU tensors: no device call)."""
    n, HK, HV = 4, 1, 2
    q = torch.zeros(n, HK, 128)
    v = torch.zeros(n, HV, 128)
    ab = torch.zeros(n, HV)
    layer_args = (q, q, v, v, ab, ab, torch.zeros(HV), torch.zeros(HV), torch.ones(128))
    cu = torch.tensor([0, 4], dtype=torch.int32)
    si = torch.arange(4, dtype=torch.int32).reshape(1, 4)
    na = torch.ones(1, dtype=torch.int32)
    idx = torch.arange(n, dtype=torch.int32)
    for bad in (torch.zeros(8, 1, 128, 128), torch.zeros(8, 4, 128, 128),
                torch.zeros(8, HV, 64, 128), torch.zeros(8, HV, 128, 64)):
        with pytest.raises(ValueError, match="the layer needs"):
            ops.spec_decode_update(*layer_args, bad, cu, si, na)
        with pytest.raises(ValueError, match="the layer needs"):
            ops.decode_update(*layer_args, bad, idx)
        with pytest.raises(ValueError, match="the layer needs"):
            ops.mixed_decode_update(*layer_args, bad, cu, si, na, idx)
        with pytest.raises(ValueError, match="the layer needs"):
            ops.prefill_update(*layer_args, bad, cu, idx[:1])
    layer = ops.make_layer(*layer_args, torch.zeros(n, HV, 128))
    assert ops.make_pool(torch.zeros(8, HV, 128, 128), layer).num_slots == 8
    # a single-token gather index needs an entry per slot entry
    pool = torch.zeros(8, HV, 128, 128)
    with pytest.raises(ValueError, match="token_indx has 3 entries"):
        ops.decode_update(*layer_args, pool, idx, token_indx=idx[:3])
    with pytest.raises(ValueError, match="non_spec_token_indx has 2 entries"):
        ops.mixed_decode_update(*layer_args, pool, cu, si, na, idx[:3],
                                non_spec_token_indx=idx[:2])


# -- metadata contract (host validator) ------------------------------------------
def _validate(batch, num_slots=None, **over):
    args = dict(cu_seqlens=batch.cu_seqlens, spec_state_indices=batch.spec_state_indices,
                num_accepted_tokens=batch.num_accepted_tokens,
                spec_token_indx=batch.spec_token_indx, state_indices=batch.state_indices,
                non_spec_token_indx=batch.non_spec_token_indx, max_q_len=batch.T)
    args.update(over)
    ops.validate_indices(batch.pool.shape[0] if num_slots is None else num_slots,
                         batch.n_tok, **args)


def test_validator_accepts_generated_workloads(lib):
    for name in ("tiny", "mtp_b32"):
        _validate(workloads.make(name))
    _validate(workloads.mixed_batch(n_non_spec=5, n_spec=4, T=3, HK=1, HV=2, K=8, V=8,
                                    act="f32", state="f32", seed=1))


@pytest.mark.parametrize("case,needle", [
    ("acc_high", "num_accepted"),
    ("acc_neg", "num_accepted"),
    ("slot_range", "outside"),
    ("dup_write", "written twice"),
    ("row_range", "row"),
    ("row_twice", "used twice"),
    ("too_long", "max_q_len"),
    ("cu_decreasing", "decreases"),
    ("cu_start", "cu_seqlens[0]"),
    ("ns_dup_spec", "written twice"),
    ("ns_slot_range", "outside"),
])
def test_validator_rejects(lib, case, needle):
    mb = workloads.mixed_batch(n_non_spec=3, n_spec=3, T=3, HK=1, HV=2, K=8, V=8,
                               act="f32", state="f32", seed=2)
    si = mb.spec_state_indices.clone()
    acc = mb.num_accepted_tokens.clone()
    cu = mb.cu_seqlens.clone()
    st = mb.spec_token_indx.clone()
    ns = mb.state_indices.clone()
    over = {}
    if case == "acc_high":
        acc[1] = 4
    elif case == "acc_neg":
        acc[0] = -1
    elif case == "slot_range":
        si[2, 1] = mb.pool.shape[0]
    elif case == "dup_write":
        si[1, 0] = si[0, 2]
    elif case == "row_range":
        st[4] = mb.n_tok
    elif case == "row_twice":
        st[4] = st[5]
    elif case == "too_long":
        over["max_q_len"] = 2
    elif case == "cu_decreasing":
        cu[2] = cu[1] - 1
    elif case == "cu_start":
        cu = cu + 1
    elif case == "ns_dup_spec":
        ns[0] = si[0, 0]
    elif case == "ns_slot_range":
        ns[2] = mb.pool.shape[0]
    with pytest.raises(ops.GdnError) as ei:
        _validate(mb, spec_state_indices=si, num_accepted_tokens=acc, cu_seqlens=cu,
                  spec_token_indx=st, state_indices=ns, **over)
    assert needle in ei.value.reason, ei.value.reason


def test_validator_rejects_cross_sequence_read():
    """A sequence that keeps fewer rows than it accepted reads a slot it does
    not write; that slot must not be written by anyone else in the batch."""
    bt = workloads.spec_batch(B=2, T=3, HK=1, HV=2, K=8, V=8, act="f32", state="f32",
                              q_lens=[1, 3], num_slots=8, seed=3)
    si = bt.spec_state_indices.clone()
    acc = torch.tensor([3, 1], dtype=torch.int32)
    _validate(bt, spec_state_indices=si, num_accepted_tokens=acc)   # fine as drawn
    si[0, 2] = si[1, 0]          # sequence 0 now reads what sequence 1 writes
    with pytest.raises(ops.GdnError) as ei:
        _validate(bt, spec_state_indices=si, num_accepted_tokens=acc)
    assert "reads slot" in ei.value.reason and "sequence 1" in ei.value.reason
    ns = torch.tensor([int(bt.spec_state_indices[0, 2])], dtype=torch.int32)
    with pytest.raises(ops.GdnError) as ei:   # ... or what a non-spec entry writes
        _validate(bt, num_accepted_tokens=acc, state_indices=ns,
                  non_spec_token_indx=torch.tensor([bt.n_tok], dtype=torch.int32))
    assert "row" in ei.value.reason
    ops.validate_indices(9, bt.n_tok + 1, cu_seqlens=bt.cu_seqlens,
                         spec_state_indices=bt.spec_state_indices, num_accepted_tokens=acc,
                         max_q_len=3, state_indices=torch.tensor([8], dtype=torch.int32),
                         non_spec_token_indx=torch.tensor([bt.n_tok], dtype=torch.int32))
    with pytest.raises(ops.GdnError) as ei:
        ops.validate_indices(9, bt.n_tok + 1, cu_seqlens=bt.cu_seqlens,
                             spec_state_indices=bt.spec_state_indices,
                             num_accepted_tokens=acc, max_q_len=3, state_indices=ns,
                             non_spec_token_indx=torch.tensor([bt.n_tok], dtype=torch.int32))
    assert "non-spec entry" in ei.value.reason


def test_validator_padding_and_identity(lib):
    # non-spec padding (-1) is skipped; identity rows need no index array
    ops.validate_indices(4, 3, state_indices=torch.tensor([0, -1, 2], dtype=torch.int32))
    with pytest.raises(ops.GdnError):
        ops.validate_indices(4, 3, state_indices=torch.tensor([0, 0, 2], dtype=torch.int32))


def test_mixed_entry_errors_and_no_op(lib):
    layer, pool, keep = _layer_and_pool()
    m = torch.zeros(16, dtype=torch.int32)
    p = ctypes.c_void_p(m.data_ptr())
    f = lib.gdn_mixed_decode_update
    args = lambda B, nt, meta=p, ns=p, mql=4: (ctypes.byref(layer), ctypes.byref(pool), meta, B,
                                               mql, meta, 4, meta, None, ns, nt, None, None)
    assert f(*args(0, 0, None, None)) == 0                  # nothing to do: no pointer read
    assert f(*args(-1, 2)) == 1 and "negative" in ops.last_error()
    assert f(*args(1, -1)) == 1
    assert f(*args(1, 0, meta=None)) == 1 and "spec metadata" in ops.last_error()
    assert f(*args(0, 2, ns=None)) == 1 and "state_indices" in ops.last_error()
    assert f(*args(1, 1, mql=9)) == 2 and "exceeds" in ops.last_error()
    assert f(*args(1, 1, mql=0)) == 1


def test_prefill_entry_errors_and_validator(lib):
    layer, pool, keep = _layer_and_pool()
    m = torch.zeros(16, dtype=torch.int32)
    p = ctypes.c_void_p(m.data_ptr())
    f = lib.gdn_prefill_update
    assert f(ctypes.byref(layer), ctypes.byref(pool), None, 0, None, None, None, 64, None) == 0
    assert f(ctypes.byref(layer), ctypes.byref(pool), p, -1, p, None, None, 64, None) == 1
    assert f(ctypes.byref(layer), ctypes.byref(pool), p, 1, p, None, None, 0, None) == 1
    assert "chunk_size" in ops.last_error()
    assert f(ctypes.byref(layer), ctypes.byref(pool), None, 1, p, None, None, 64, None) == 1
    b = workloads.make_prefill("prefill_small")
    ops.validate_prefill_indices(b.pool.shape[0], b.n_tok, b.cu_seqlens, b.state_indices)
    si = b.state_indices.clone()
    si[3] = si[0]
    with pytest.raises(ops.GdnError) as ei:
        ops.validate_prefill_indices(b.pool.shape[0], b.n_tok, b.cu_seqlens, si)
    assert "two sequences" in ei.value.reason
    si[3] = b.pool.shape[0]
    with pytest.raises(ops.GdnError):
        ops.validate_prefill_indices(b.pool.shape[0], b.n_tok, b.cu_seqlens, si)
    tix = torch.arange(b.n_tok, dtype=torch.int32)
    tix[5] = tix[6]
    with pytest.raises(ops.GdnError) as ei:
        ops.validate_prefill_indices(b.pool.shape[0], b.n_tok, b.cu_seqlens, b.state_indices,
                                     token_indx=tix)
    assert "used twice" in ei.value.reason


def test_offset_norm_weight_view_is_rejected(lib):
    """w[1:] of a float32 tensor passes the binding's contiguity check but is
    only 4-byte aligned; the library rejects it before enqueueing anything."""
    layer, pool, keep = _layer_and_pool()
    w = torch.ones(129)[1:]
    assert w.is_contiguous() and w.data_ptr() % 8 == 4
    q, k, v, z, a, b, out, A_log, dt = keep[:9]
    layer = ops.make_layer(q, k, v, z, a, b, A_log, dt, w, out)
    assert _spec(lib, layer, pool) == 1
    assert "norm_weight must be 8-byte" in ops.last_error()


def test_traffic_pattern_argument_errors(lib):
    """The measurement entry runs the same host checks as the update entries
    and enqueues nothing when they fail (CPU tensors: no device call)."""
    layer, pool, keep = _layer_and_pool()
    m = torch.zeros(16, dtype=torch.int32)
    p = ctypes.c_void_p(m.data_ptr())
    call = lambda L, B, maxq, ns: lib.gdn_traffic_pattern(   # noqa: E731
        ctypes.byref(L), ctypes.byref(pool), p, B, maxq, p, 4, p, None, p, ns, None, 0, None)
    assert call(layer, 0, 4, 0) == 0                         # nothing to do
    assert call(layer, 1, 9, 0) == 2 and "exceeds" in ops.last_error()
    assert call(layer, -1, 4, 0) == 1
    assert lib.gdn_traffic_pattern(ctypes.byref(layer), ctypes.byref(pool), p, 1, 4, p, 4, p,
                                   None, p, 0, None, 9, None) == 1
    assert "blocks_per_cu" in ops.last_error()
    layer.norm_weight = layer.norm_weight + 4
    assert call(layer, 1, 4, 0) == 1 and "norm_weight" in ops.last_error()


def test_issue_probe_argument_errors(lib):
    """The issue probe checks its arguments on the host and enqueues nothing
    when they fail (no device call here)."""
    out = ctypes.c_void_p(0x1000)          # never dereferenced: every call fails first
    assert lib.gdn_issue_probe(None, 1, 1, 1, 1, None) == 1 and "NULL" in ops.last_error()
    assert lib.gdn_issue_probe(out, 1, 0, 1, 1, None) == 1 and "mode" in ops.last_error()
    assert lib.gdn_issue_probe(out, 1, 4, 1, 1, None) == 1
    assert lib.gdn_issue_probe(out, 0, 3, 1, 1, None) == 1 and "blocks" in ops.last_error()
    assert lib.gdn_issue_probe(out, 65537, 3, 1, 1, None) == 1
    assert lib.gdn_issue_probe(out, 1, 3, -1, 1, None) == 1 and "chain" in ops.last_error()
    assert lib.gdn_issue_probe(out, 1, 3, 1, 1000001, None) == 1
