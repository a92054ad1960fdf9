"""CPU checks of the C ABI: the library loads, exports every function that
include/attn.h declares, its host-side frequency tables agree with the oracle,
and argument validation returns the documented status before any launch."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from chunked_prefill_causal_rope_amd import api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

OK, EINVAL, ECAP, EUNSUP = 0, -1, -2, -3


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = api.lib()
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), f"{n} declared in attn.h but not exported"
    assert set(api.EXPORTS) <= set(names)
    assert L.attn_version().decode().count(".") == 2


def test_status_strings():
    L = api.lib()
    for code in (OK, EINVAL, ECAP, EUNSUP, -4):
        assert L.attn_status_string(code).decode() != "unknown status"
    assert L.attn_status_string(123).decode() == "unknown status"


@pytest.mark.parametrize("rd,base", [(4, 1e4), (64, 1e4), (128, 1e4), (64, 1e6), (128, 5e5), (32, 500.0)])
def test_rope_table_matches_oracle(rd, base):
    got = api.rope_inv_freq(rd, base).numpy()
    ref = oracle.rope_inv_freq(rd, base)
    ulps = np.abs(got.view(np.int32).astype(np.int64) - ref.view(np.int32).astype(np.int64))
    assert ulps.max() <= 1, ulps.max()


@pytest.mark.parametrize("args", [
    (64, 5e5, 128.0, 8192, 32.0, 1.0),
    (128, 1e6, 4.0, 32768, 32.0, 1.0),
    (64, 1e4, 8.0, 4096, 32.0, 1.0),
    (128, 1e4, 2.0, 2048, 16.0, 2.0),
])
def test_yarn_table_matches_oracle(args):
    got = api.yarn_inv_freq(*args).numpy()
    ref = oracle.yarn_inv_freq(*args)
    ulps = np.abs(got.view(np.int32).astype(np.int64) - ref.view(np.int32).astype(np.int64))
    assert ulps.max() <= 1, ulps.max()


def test_table_argument_errors():
    L = api.lib()
    buf = (ctypes.c_float * 64)()
    assert L.attn_rope_inv_freq(7, 1e4, buf) == EINVAL
    assert L.attn_rope_inv_freq(0, 1e4, buf) == EINVAL
    assert L.attn_rope_inv_freq(64, -1.0, buf) == EINVAL
    assert L.attn_rope_inv_freq(64, 1e4, None) == EINVAL
    assert L.attn_yarn_inv_freq(64, 1e4, 0.0, 4096, 32.0, 1.0, buf) == EINVAL
    assert L.attn_yarn_inv_freq(64, 1e4, 4.0, 0, 32.0, 1.0, buf) == EINVAL


# A fake device address: the validation paths below return before any HIP
# call, so it is never dereferenced.
P = ctypes.c_void_p(4096)


def prefill(**kw):
    a = dict(q=P, k=P, v=P, dtype=1, n_seq=1, nh=8, nkv=2, hd=128, cap=256, ring=0, n_tok=16, cu=P, st=P,
             max_chunk=16, max_end=64, scale=0.088, window=0, gate=None, gate_mode=0, gate_ld=0,
             out=P, ws=None, wsb=0, stream=None)
    a.update(kw)
    return api.lib().attn_prefill_chunk(a["q"], a["k"], a["v"], a["dtype"], a["n_seq"], a["nh"],
                                        a["nkv"], a["hd"], a["cap"], a["ring"], a["n_tok"], a["cu"], a["st"],
                                        a["max_chunk"], a["max_end"], a["scale"], a["window"],
                                        a["gate"], a["gate_mode"], a["gate_ld"],
                                        a["out"], a["ws"], a["wsb"], a["stream"])


def test_prefill_validation():
    assert prefill(hd=96) == EUNSUP
    assert prefill(dtype=5) == EUNSUP
    assert prefill(nh=6, nkv=4) == EINVAL
    assert prefill(nkv=0) == EINVAL
    assert prefill(max_end=257) == ECAP
    assert prefill(scale=float("nan")) == EINVAL
    assert prefill(window=-1) == EINVAL
    assert prefill(ring=2) == EINVAL
    # output gates: a mode needs a gate, per-element modes a full row
    assert prefill(gate_mode=1) == EINVAL
    assert prefill(gate_mode=4, gate=P, gate_ld=128) == EINVAL
    assert prefill(gate_mode=1, gate=P, gate_ld=127) == EINVAL
    assert prefill(gate_mode=2, gate=P, gate_ld=0) == EINVAL
    assert prefill(gate_mode=2, gate=P, gate_ld=1, n_tok=0) == OK
    # a ring that has wrapped needs a window, and window + max_chunk - 1 rows
    assert prefill(ring=1, max_end=300) == ECAP
    assert prefill(ring=1, max_end=300, window=250) == ECAP
    # bf16 ring rows come in whole 64-key tiles
    assert prefill(ring=1, max_end=300, window=100, cap=200) == EUNSUP
    assert prefill(q=None) == EINVAL
    assert prefill(cu=None) == EINVAL
    # empty work: OK and nothing launched
    assert prefill(n_tok=0) == OK
    assert prefill(n_seq=0) == OK
    assert prefill(max_chunk=0) == OK


def append(**kw):
    a = dict(kc=P, vc=P, dtype=1, n_seq=1, nkv=2, hd=128, cap=256, ring=0, kn=P, vn=P, n_tok=16, cu=P,
             st=P, max_chunk=16, max_end=64, f=P, rd=128, rs=1.0, norm=0, w=None, eps=1e-6, v_norm=0)
    a.update(kw)
    return api.lib().attn_kv_append(a["kc"], a["vc"], a["dtype"], a["n_seq"], a["nkv"], a["hd"],
                                    a["cap"], a["ring"], a["kn"], a["vn"], a["n_tok"], a["cu"], a["st"],
                                    a["max_chunk"], a["max_end"], a["f"], a["rd"], a["rs"],
                                    a["norm"], a["w"], a["eps"], a["v_norm"], None)


def test_append_validation():
    assert append(max_end=300) == ECAP
    assert append(ring=3) == EINVAL
    assert append(v_norm=2) == EINVAL
    assert append(ring=1, max_end=300, n_seq=0) == OK     # a ring has a row for every position
    # a wrapped ring shorter than the chunk would give p and p + cap one row
    assert append(ring=1, max_end=600, max_chunk=257, n_tok=257) == ECAP
    assert append(ring=1, max_end=600, max_chunk=256, n_tok=256, n_seq=0) == OK
    assert append(rd=63) == EINVAL
    assert append(f=None) == EINVAL
    assert append(norm=1, w=None) == EINVAL
    assert append(norm=3, w=P) == EINVAL
    assert append(hd=80) == EUNSUP
    assert append(cap=0) == EINVAL
    assert append(n_tok=0) == OK
    assert append(rd=0, f=None, n_seq=0) == OK


def rope_qkv(**kw):
    a = dict(q=P, qo=P, nh=8, kc=P, vc=P, kn=P, vn=P, nkv=2, cap=256, ring=0, dtype=1, n_tok=16, hd=128,
             n_seq=1, cu=P, st=P, max_chunk=16, max_end=64, f=P, rd=128, rs=1.0, norm=0, qw=None,
             kw=None, eps=1e-6, v_norm=0)
    a.update(kw)
    return api.lib().attn_rope_qkv(a["q"], a["qo"], a["nh"], a["kc"], a["vc"], a["kn"], a["vn"], a["nkv"],
                                   a["cap"], a["ring"], a["dtype"], a["n_tok"], a["hd"], a["n_seq"],
                                   a["cu"], a["st"], a["max_chunk"], a["max_end"], a["f"], a["rd"],
                                   a["rs"], a["norm"], a["qw"], a["kw"], a["eps"], a["v_norm"], None)


def test_rope_qkv_validation():
    assert rope_qkv(max_end=300) == ECAP
    assert rope_qkv(ring=1, max_end=600, max_chunk=257, n_tok=257) == ECAP
    assert rope_qkv(ring=1, max_end=600, max_chunk=256, n_tok=256, n_seq=0) == OK
    assert rope_qkv(ring=2) == EINVAL
    assert rope_qkv(norm=1, qw=P, kw=None) == EINVAL
    assert rope_qkv(nkv=0) == EINVAL
    assert rope_qkv(hd=96) == EUNSUP
    assert rope_qkv(q=None) == EINVAL
    assert rope_qkv(n_tok=0) == OK


def prefill_rope_next(nxt, **kw):
    """attn_prefill_chunk_rope_next with prefill()'s defaults; nxt: rope_qkv()'s
    keyword overrides for the next chunk, or None for a NULL next."""
    a = dict(q=P, k=P, v=P, dtype=1, n_seq=1, nh=8, nkv=2, hd=128, cap=256, ring=0, n_tok=16, cu=P, st=P,
             max_chunk=16, max_end=64, scale=0.088, window=0, gate=None, gate_mode=0, gate_ld=0,
             out=P, ws=None, wsb=0, stream=None)
    a.update(kw)
    ptr = None
    if nxt is not None:
        r = dict(q=P, q_out=P, n_heads=8, k_cache=P, v_cache=P, k_new=P, v_new=P, n_kv=2, cap=256, ring=0,
                 dtype=1, n_tok=16, head_dim=128, n_seq=1, cu_seq=P, start=P, max_chunk=16, max_end=80,
                 inv_freq=P, rotary_dim=128, rope_scale=1.0, norm=0, q_norm_w=None, k_norm_w=None, eps=1e-6,
                 v_norm=0)
        r.update(nxt)
        r = {k: (v.value if isinstance(v, ctypes.c_void_p) else v) for k, v in r.items()}
        ptr = ctypes.byref(api.RopeQkvArgs(**r))
    return api.lib().attn_prefill_chunk_rope_next(
        a["q"], a["k"], a["v"], a["dtype"], a["n_seq"], a["nh"], a["nkv"], a["hd"], a["cap"], a["ring"],
        a["n_tok"], a["cu"], a["st"], a["max_chunk"], a["max_end"], a["scale"], a["window"], a["gate"],
        a["gate_mode"], a["gate_ld"], a["out"], a["ws"], a["wsb"], ptr, a["stream"])


def test_prefill_rope_next_validation():
    # every error of either call comes back before anything is launched
    assert prefill_rope_next(None) == EINVAL
    assert prefill_rope_next({"max_end": 300}) == ECAP          # the next chunk's append
    assert prefill_rope_next({"head_dim": 96}) == EUNSUP
    assert prefill_rope_next({"q": None}) == EINVAL
    assert prefill_rope_next({}, max_end=257) == ECAP            # this chunk's attention
    assert prefill_rope_next({}, hd=96) == EUNSUP
    assert prefill_rope_next({}, window=-1) == EINVAL
    assert prefill_rope_next({}, gate_mode=1) == EINVAL
    # no work in either call: OK, nothing launched
    assert prefill_rope_next({"n_tok": 0}, n_tok=0) == OK
    assert prefill_rope_next({"n_seq": 0}, n_seq=0) == OK


def prefill_deferred(nxt, prev=None, pending="new", **kw):
    """attn_prefill_chunk_deferred with prefill_rope_next()'s defaults; nxt as
    there (None: no next chunk); prev / pending: PrefillPending records (or
    None for NULL; pending defaults to a fresh record)."""
    a = dict(q=P, k=P, v=P, dtype=1, n_seq=1, nh=8, nkv=2, hd=128, cap=256, ring=0, n_tok=16, cu=P, st=P,
             max_chunk=16, max_end=64, scale=0.088, window=0, gate=None, gate_mode=0, gate_ld=0,
             out=P, ws=None, wsb=0, stream=None)
    a.update(kw)
    ptr = None
    if nxt is not None:
        r = dict(q=P, q_out=P, n_heads=8, k_cache=P, v_cache=P, k_new=P, v_new=P, n_kv=2, cap=256, ring=0,
                 dtype=1, n_tok=16, head_dim=128, n_seq=1, cu_seq=P, start=P, max_chunk=16, max_end=80,
                 inv_freq=P, rotary_dim=128, rope_scale=1.0, norm=0, q_norm_w=None, k_norm_w=None, eps=1e-6,
                 v_norm=0)
        r.update(nxt)
        r = {k: (v.value if isinstance(v, ctypes.c_void_p) else v) for k, v in r.items()}
        ptr = ctypes.byref(api.RopeQkvArgs(**r))
    if isinstance(pending, str):
        pending = api.PrefillPending()
    return api.lib().attn_prefill_chunk_deferred(
        a["q"], a["k"], a["v"], a["dtype"], a["n_seq"], a["nh"], a["nkv"], a["hd"], a["cap"], a["ring"],
        a["n_tok"], a["cu"], a["st"], a["max_chunk"], a["max_end"], a["scale"], a["window"], a["gate"],
        a["gate_mode"], a["gate_ld"], a["out"], a["ws"], a["wsb"], ptr,
        ctypes.byref(prev) if prev is not None else None,
        ctypes.byref(pending) if pending is not None else None, a["stream"])


def test_prefill_deferred_validation():
    L = api.lib()
    assert prefill_deferred(None, pending=None) == EINVAL
    # every error of the chunk and of the next chunk's finish, before any launch
    assert prefill_deferred({"max_end": 300}) == ECAP
    assert prefill_deferred({"head_dim": 96}) == EUNSUP
    assert prefill_deferred(None, max_end=257) == ECAP
    assert prefill_deferred(None, hd=96) == EUNSUP
    assert prefill_deferred(None, gate_mode=1) == EINVAL
    # a record the library did not write
    bad = api.PrefillPending()
    bad.active = 2
    assert prefill_deferred(None, prev=bad) == EINVAL
    assert L.attn_prefill_finish(ctypes.byref(bad), None) == EINVAL
    bad.active, bad.head_dim = 1, 96
    assert prefill_deferred(None, prev=bad) == EINVAL
    assert L.attn_prefill_finish(ctypes.byref(bad), None) == EINVAL
    # active with a valid head size, but not written by the library (its
    # check word does not match): refused before anything could launch
    bad.head_dim = 128
    assert prefill_deferred(None, prev=bad) == EINVAL
    assert L.attn_prefill_finish(ctypes.byref(bad), None) == EINVAL
    assert L.attn_prefill_finish(None, None) == EINVAL
    # nothing owed, nothing to run: OK without a launch, and the record says so
    rec = api.PrefillPending()
    rec.active = 1
    assert prefill_deferred(None, pending=rec, n_seq=0) == OK and rec.active == 0 and rec.head_dim == 128
    assert prefill_deferred({"n_tok": 0}, prev=rec, pending=rec, n_tok=0) == OK and rec.active == 0
    assert L.attn_prefill_finish(ctypes.byref(rec), None) == OK


def test_pipelined_buffers_must_be_disjoint():
    """The pipelined calls run the next chunk's finish (and a deferred merge)
    beside this chunk's attention: a buffer one of them writes may not overlap
    one another reads or writes.  Refused before anything is launched."""
    def at(mb):
        return ctypes.c_void_p(mb << 20)
    # this chunk: q at 16 MB, out at 32 MB; next: q at 48, q_out at 64, k/v at 80 and 96 MB
    mine = dict(q=at(16), out=at(32))
    nxt = dict(q=at(48), q_out=at(64), k_new=at(80), v_new=at(96))
    clash = [({**nxt, "q_out": at(16)}, {}),                 # next's queries written over this q
             ({**nxt, "q_out": at(32)}, {}),                 # ... over this chunk's output
             ({**nxt, "q": at(32)}, {}),                     # next reads rows this chunk writes
             ({**nxt, "v_new": ctypes.c_void_p((32 << 20) + 4096)}, {}),
             (nxt, {"ws": at(64), "wsb": 4096}),             # workspace over next's rotated queries
             ({**nxt, "q_out": at(200)}, {"gate": ctypes.c_void_p((200 << 20) - 64), "gate_mode": 1,
                                          "gate_ld": 128})]  # the gate rows' tail
    for n, extra in clash:
        assert prefill_rope_next(n, **mine, **extra) == EINVAL
        assert prefill_deferred(n, **mine, **extra) == EINVAL


def rope(**kw):
    a = dict(x=P, y=P, dtype=0, n_tok=4, nh=4, hd=64, n_seq=1, cu=P, st=P, max_chunk=4, f=P,
             rd=64, rs=1.0, norm=0, w=None, eps=1e-6)
    a.update(kw)
    return api.lib().attn_rope_apply(a["x"], a["y"], a["dtype"], a["n_tok"], a["nh"], a["hd"],
                                     a["n_seq"], a["cu"], a["st"], a["max_chunk"], a["f"], a["rd"],
                                     a["rs"], a["norm"], a["w"], a["eps"], None)


def test_rope_validation():
    assert rope(hd=48) == EUNSUP
    assert rope(nh=0) == EINVAL
    assert rope(rd=3) == EINVAL
    assert rope(n_tok=-1) == EINVAL
    assert rope(x=None) == EINVAL
    assert rope(norm=2, w=None) == EINVAL
    assert rope(n_seq=0) == OK
    assert rope(max_chunk=0) == OK


def decode(**kw):
    a = dict(q=P, k=P, v=P, dtype=1, n_seq=4, nh=32, nkv=8, hd=128, cap=4096, ring=0, ctx=P, max_ctx=4096,
             scale=0.088, window=0, gate=None, gate_mode=0, gate_ld=0, out=P, probs=None, ld=0, ws=P,
             wsb=1 << 30)
    a.update(kw)
    return api.lib().attn_decode(a["q"], a["k"], a["v"], a["dtype"], a["n_seq"], a["nh"],
                                 a["nkv"], a["hd"], a["cap"], a["ring"], a["ctx"], a["max_ctx"], a["scale"],
                                 a["window"], a["gate"], a["gate_mode"], a["gate_ld"], a["out"],
                                 a["probs"], a["ld"], a["ws"], a["wsb"], None)


def test_decode_validation():
    assert decode(max_ctx=4097) == ECAP
    assert decode(probs=P, ld=100) == EINVAL
    assert decode(nh=34) == EINVAL
    assert decode(nh=64, nkv=2) == EUNSUP        # 32 query heads per KV head
    assert decode(ws=None, wsb=0) == EINVAL      # bf16 needs a workspace
    assert decode(wsb=16) == EINVAL
    assert decode(hd=256) == EUNSUP
    assert decode(window=-5) == EINVAL
    assert decode(ring=-1) == EINVAL
    assert decode(gate_mode=3, gate=None, gate_ld=128) == EINVAL
    assert decode(gate_mode=3, gate=P, gate_ld=64) == EINVAL
    # a wrapped ring holds the last cap keys: 0 < window <= cap
    assert decode(ring=1, max_ctx=5000, probs=P, ld=5000) == ECAP
    assert decode(ring=1, max_ctx=5000, window=4097) == ECAP
    assert decode(n_seq=0) == OK
    assert decode(max_ctx=0) == OK


def test_workspace_sizes():
    L = api.lib()
    # decode: one part per 1024 keys, each a 16-byte header and head_dim halves
    assert L.attn_decode_workspace_bytes(64, 32, 8, 128, 32768) == 64 * 32 * 32 * (16 + 2 * 128)
    assert L.attn_decode_workspace_bytes(0, 32, 8, 128, 32768) == 0
    # prefill: a large grid needs no split
    assert L.attn_prefill_workspace_bytes(1, 64, 8, 128, 2048, 2048, 4096) == 0
    # a small chunk over a long context splits the key range: a 256-byte
    # table, then one partial (128 rows of a 16-byte header and 128 halves)
    # per work item
    n = L.attn_prefill_workspace_bytes(1, 32, 8, 128, 128, 128, 4096)
    assert n > 256 and (n - 256) % (128 * (16 + 2 * 128)) == 0


def importance(**kw):
    a = dict(probs=P, n_seq=4, nh=32, ld=4096, ctx=P, max_ctx=4096, imp=P, imp_ld=4096, acc=1)
    a.update(kw)
    return api.lib().attn_decode_importance(a["probs"], a["n_seq"], a["nh"], a["ld"], a["ctx"],
                                            a["max_ctx"], a["imp"], a["imp_ld"], a["acc"], None)


def test_importance_validation():
    assert importance(probs=None) == EINVAL
    assert importance(imp=None) == EINVAL
    assert importance(ctx=None) == EINVAL
    assert importance(ld=4095) == EINVAL
    assert importance(imp_ld=100) == EINVAL
    assert importance(nh=0) == EINVAL
    assert importance(n_seq=-1) == EINVAL
    assert importance(n_seq=0) == OK
    assert importance(max_ctx=0) == OK


def test_calibration_validation():
    L = api.lib()
    P = ctypes.c_void_p(0x1000)        # never dereferenced: every call fails validation
    assert L.attn_calibrate_mfma(0, 10, 1, P, None) == EINVAL
    assert L.attn_calibrate_mfma(4, 0, 0, P, None) == EINVAL
    assert L.attn_calibrate_mfma(4, 10, 2, P, None) == EINVAL
    assert L.attn_calibrate_mfma(4, 10, -1, P, None) == EINVAL
    assert L.attn_calibrate_mfma(4, 10, 1, None, None) == EINVAL
    assert L.attn_calibrate_read(P, 15, 4, P, None) == EINVAL
    assert L.attn_calibrate_read(P, 1 << 20, 0, P, None) == EINVAL
    assert L.attn_calibrate_read(ctypes.c_void_p(0x1008), 1 << 20, 4, P, None) == EINVAL
    assert L.attn_calibrate_read(None, 1 << 20, 4, P, None) == EINVAL


def test_recorded_traffic_keyed_to_the_built_code():
    """bench.py reports counter traffic only for the GPU code it was taken on:
    the key is a hash of the built library's .hip_fatbin section, and a record
    under another key reads as absent."""
    import json
    import bench
    code = bench.kernel_code_hash()
    assert code is not None and re.fullmatch(r"[0-9a-f]{16}", code)
    assert bench.kernel_code_hash() == code          # deterministic
    rec = json.load(open(os.path.join(os.path.dirname(os.path.dirname(__file__)), "profiles", "traffic.json")))
    for name, w in rec["workloads"].items():
        want = w["bytes_per_launch"] if rec.get("kernel_code_hash") == code else None
        assert bench.recorded_traffic(name) == want
    assert bench.recorded_traffic("no_such_workload") is None
