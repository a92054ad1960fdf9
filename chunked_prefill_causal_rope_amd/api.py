"""Thin ctypes binding of libattn.so (the C ABI in include/attn.h).

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, then their device pointers and the current torch stream are handed
to the library.  Every step of the path runs in the library's HIP kernels; if
the library is missing this module raises, it never computes anything itself.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libattn.so")

F32, BF16 = 0, 1
NORM_NONE, NORM_W, NORM_1PW = 0, 1, 2
_STATUS = {0: "ok", -1: "invalid argument", -2: "exceeds cache capacity",
           -3: "unsupported configuration", -4: "device launch failed",
           -5: "exceeds the library's static scratch"}

_lib = None

EXPORTS = ("attn_rope_inv_freq", "attn_yarn_inv_freq", "attn_rope_apply", "attn_kv_append",
           "attn_rope_qkv", "attn_prefill_chunk", "attn_prefill_chunk_rope_next",
           "attn_prefill_chunk_deferred", "attn_prefill_finish",
           "attn_prefill_workspace_bytes", "attn_decode",
           "attn_decode_workspace_bytes", "attn_decode_importance", "attn_calibrate_mfma",
           "attn_calibrate_read", "attn_status_string", "attn_version")


class RopeQkvArgs(ctypes.Structure):
    """attn_rope_qkv_args of attn.h (field for field)."""
    _fields_ = [("q", ctypes.c_void_p), ("q_out", ctypes.c_void_p), ("n_heads", ctypes.c_int),
                ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p), ("k_new", ctypes.c_void_p),
                ("v_new", ctypes.c_void_p), ("n_kv", ctypes.c_int), ("cap", ctypes.c_int), ("ring", ctypes.c_int),
                ("dtype", ctypes.c_int), ("n_tok", ctypes.c_int), ("head_dim", ctypes.c_int),
                ("n_seq", ctypes.c_int), ("cu_seq", ctypes.c_void_p), ("start", ctypes.c_void_p),
                ("max_chunk", ctypes.c_int), ("max_end", ctypes.c_int), ("inv_freq", ctypes.c_void_p),
                ("rotary_dim", ctypes.c_int), ("rope_scale", ctypes.c_float), ("norm", ctypes.c_int),
                ("q_norm_w", ctypes.c_void_p), ("k_norm_w", ctypes.c_void_p), ("eps", ctypes.c_double),
                ("v_norm", ctypes.c_int)]


class PrefillPending(ctypes.Structure):
    """attn_prefill_pending of attn.h: a split chunk's merge owed to a later
    launch (active), the rest the library's."""
    _fields_ = [("active", ctypes.c_int), ("head_dim", ctypes.c_int), ("state", ctypes.c_uint64 * 16)]


class AttnError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {_STATUS.get(status, 'unknown status')} ({status})")
        self.status = status


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build() first "
                           "(there is no fallback implementation)")
    L = ctypes.CDLL(LIB_PATH)
    i, d, f, vp, sz = ctypes.c_int, ctypes.c_double, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
    fp = ctypes.POINTER(ctypes.c_float)
    L.attn_rope_inv_freq.argtypes = [i, d, fp]
    L.attn_yarn_inv_freq.argtypes = [i, d, d, i, d, d, fp]
    L.attn_rope_apply.argtypes = [vp, vp, i, i, i, i, i, vp, vp, i, vp, i, f, i, vp, d, vp]
    L.attn_kv_append.argtypes = [vp, vp, i, i, i, i, i, i, vp, vp, i, vp, vp, i, i, vp, i, f, i,
                                 vp, d, i, vp]
    L.attn_rope_qkv.argtypes = [vp, vp, i, vp, vp, vp, vp, i, i, i, i, i, i, i, vp, vp, i, i, vp, i,
                                f, i, vp, vp, d, i, vp]
    L.attn_prefill_chunk.argtypes = [vp, vp, vp, i, i, i, i, i, i, i, i, vp, vp, i, i, f, i, vp, i,
                                     i, vp, vp, sz, vp]
    L.attn_prefill_chunk_rope_next.argtypes = [vp, vp, vp, i, i, i, i, i, i, i, i, vp, vp, i, i, f, i,
                                               vp, i, i, vp, vp, sz, ctypes.POINTER(RopeQkvArgs), vp]
    pend = ctypes.POINTER(PrefillPending)
    L.attn_prefill_chunk_deferred.argtypes = [vp, vp, vp, i, i, i, i, i, i, i, i, vp, vp, i, i, f, i,
                                              vp, i, i, vp, vp, sz, ctypes.POINTER(RopeQkvArgs), pend, pend,
                                              vp]
    L.attn_prefill_finish.argtypes = [pend, vp]
    L.attn_prefill_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
    L.attn_prefill_workspace_bytes.restype = sz
    L.attn_decode.argtypes = [vp, vp, vp, i, i, i, i, i, i, i, vp, i, f, i, vp, i, i, vp, vp, i, vp,
                              sz, vp]
    L.attn_decode_workspace_bytes.argtypes = [i, i, i, i, i]
    if hasattr(L, "attn_decode_noalloc"):
        L.attn_decode_noalloc.argtypes = [vp, vp, vp, i, i, i, i, i, i, i, vp, i, f, i, vp, i, i, vp,
                                          vp, i, vp]
        L.attn_decode_noalloc.restype = i
    L.attn_decode_importance.argtypes = [vp, i, i, i, vp, i, vp, i, i, vp]
    L.attn_decode_importance.restype = i
    L.attn_decode_workspace_bytes.restype = sz
    L.attn_calibrate_mfma.argtypes = [i, i, i, vp, vp]
    L.attn_calibrate_mfma.restype = i
    L.attn_calibrate_read.argtypes = [vp, sz, i, vp, vp]
    L.attn_calibrate_read.restype = i
    L.attn_status_string.argtypes = [i]
    L.attn_status_string.restype = ctypes.c_char_p
    L.attn_version.restype = ctypes.c_char_p
    for name in ("attn_rope_inv_freq", "attn_yarn_inv_freq", "attn_rope_apply", "attn_kv_append",
                 "attn_rope_qkv", "attn_prefill_chunk", "attn_prefill_chunk_rope_next",
                 "attn_prefill_chunk_deferred", "attn_prefill_finish", "attn_decode"):
        getattr(L, name).restype = i
    _lib = L
    return L


def _check(fn: str, st: int):
    if st != 0:
        raise AttnError(fn, st)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(t: torch.Tensor | None, name: str, dtype=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


GATE_NONE, GATE_SIGMOID, GATE_SOFTPLUS_HEAD, GATE_SOFTPLUS = 0, 1, 2, 3


def _gate(gate: torch.Tensor | None, mode: int, n_rows: int, n_heads: int, head_dim: int, dtype):
    """(pointer, mode, gate_ld) of an output gate: [n_rows][n_heads][>= head_dim]
    per element, [n_rows][n_heads] (or [..][..][1+]) per head; the innermost
    dim must be contiguous and the heads evenly strided (a view of the raw
    query projection's second halves is fine)."""
    if mode == GATE_NONE or gate is None:
        return None, GATE_NONE, 0
    if not gate.is_cuda or gate.dtype != dtype:
        raise ValueError("gate must be a device tensor of the call's dtype")
    g = gate if gate.dim() == 3 else gate.unsqueeze(-1)
    assert g.shape[0] >= n_rows and g.shape[1] == n_heads
    assert g.stride(-1) == 1 or g.shape[-1] == 1
    ld = g.stride(1)
    assert g.stride(0) == n_heads * ld, "heads must be evenly strided across rows"
    if mode != GATE_SOFTPLUS_HEAD:
        assert g.shape[2] >= head_dim
    return g.data_ptr(), mode, ld


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


# ---------------------------------------------------------------- tables

def rope_inv_freq(rotary_dim: int, base: float) -> torch.Tensor:
    out = torch.zeros(rotary_dim // 2, dtype=torch.float32)
    _check("attn_rope_inv_freq", lib().attn_rope_inv_freq(
        rotary_dim, base, ctypes.cast(out.data_ptr(), ctypes.POINTER(ctypes.c_float))))
    return out


def yarn_inv_freq(rotary_dim: int, base: float, factor: float, orig_max_pos: int,
                  beta_fast: float, beta_slow: float) -> torch.Tensor:
    out = torch.zeros(rotary_dim // 2, dtype=torch.float32)
    _check("attn_yarn_inv_freq", lib().attn_yarn_inv_freq(
        rotary_dim, base, factor, orig_max_pos, beta_fast, beta_slow,
        ctypes.cast(out.data_ptr(), ctypes.POINTER(ctypes.c_float))))
    return out


# ---------------------------------------------------------------- batch descriptor

class Batch:
    """Varlen descriptor: sequences b = 0..n_seq-1 contribute lens[b] packed
    rows starting at absolute position starts[b]."""

    def __init__(self, starts: list[int], lens: list[int], device="cuda"):
        assert len(starts) == len(lens)
        self.starts = [int(s) for s in starts]
        self.lens = [int(n) for n in lens]
        cu = [0]
        for n in self.lens:
            cu.append(cu[-1] + n)
        self.cu_list = cu
        self.n_seq = len(lens)
        self.n_tok = cu[-1]
        self.max_chunk = max(self.lens) if self.lens else 0
        self.max_end = max((s + n for s, n in zip(self.starts, self.lens)), default=0)
        self.cu_seq = torch.tensor(cu, dtype=torch.int32, device=device)
        self.start = torch.tensor(self.starts or [0], dtype=torch.int32, device=device)


# ---------------------------------------------------------------- entry points

def rope_apply(x: torch.Tensor, y: torch.Tensor, batch: Batch, inv_freq: torch.Tensor,
               rotary_dim: int, rope_scale: float = 1.0, norm: int = NORM_NONE,
               norm_w: torch.Tensor | None = None, eps: float = 1e-6):
    n_tok, n_heads, hd = x.shape
    assert y.shape == x.shape and y.dtype == x.dtype and n_tok >= batch.n_tok
    st = lib().attn_rope_apply(
        _dev(x, "x"), _dev(y, "y"), _dtype_code(x), n_tok, n_heads, hd, batch.n_seq,
        _dev(batch.cu_seq, "cu_seq", torch.int32), _dev(batch.start, "start", torch.int32),
        batch.max_chunk, _dev(inv_freq, "inv_freq", torch.float32) if rotary_dim else None,
        rotary_dim, rope_scale, norm, _dev(norm_w, "norm_w", torch.float32), eps, _stream())
    _check("attn_rope_apply", st)


def kv_append(k_cache: torch.Tensor, v_cache: torch.Tensor, k_new: torch.Tensor,
              v_new: torch.Tensor, batch: Batch, inv_freq: torch.Tensor, rotary_dim: int,
              rope_scale: float = 1.0, norm: int = NORM_NONE,
              norm_w: torch.Tensor | None = None, eps: float = 1e-6, ring: bool = False,
              v_norm: bool = False):
    """Finish K rows and write them with the V rows at their positions (row
    p mod cap with ring=True); v_norm RMS-normalises the V rows first."""
    n_seq_c, n_kv, cap, hd = k_cache.shape
    assert v_cache.shape == k_cache.shape and n_seq_c >= batch.n_seq
    n_tok = k_new.shape[0]
    assert k_new.shape == (n_tok, n_kv, hd) and v_new.shape == k_new.shape
    assert k_new.dtype == k_cache.dtype == v_cache.dtype == v_new.dtype
    st = lib().attn_kv_append(
        _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dtype_code(k_cache), batch.n_seq,
        n_kv, hd, cap, int(ring), _dev(k_new, "k_new"), _dev(v_new, "v_new"), n_tok,
        _dev(batch.cu_seq, "cu_seq", torch.int32), _dev(batch.start, "start", torch.int32),
        batch.max_chunk, batch.max_end,
        _dev(inv_freq, "inv_freq", torch.float32) if rotary_dim else None, rotary_dim,
        rope_scale, norm, _dev(norm_w, "norm_w", torch.float32), eps, int(v_norm), _stream())
    _check("attn_kv_append", st)


def rope_qkv(q: torch.Tensor, q_out: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
             k_new: torch.Tensor, v_new: torch.Tensor, batch: Batch, inv_freq: torch.Tensor,
             rotary_dim: int, rope_scale: float = 1.0, norm: int = NORM_NONE,
             q_norm_w: torch.Tensor | None = None, k_norm_w: torch.Tensor | None = None,
             eps: float = 1e-6, ring: bool = False, v_norm: bool = False):
    """rope_apply(q -> q_out) and kv_append(k_new, v_new) of one chunk in one call."""
    st = lib().attn_rope_qkv(*_rope_qkv_args(q, q_out, k_cache, v_cache, k_new, v_new, batch, inv_freq,
                                             rotary_dim, rope_scale, norm, q_norm_w, k_norm_w, eps, ring,
                                             v_norm), _stream())
    _check("attn_rope_qkv", st)


def _rope_qkv_args(q, q_out, k_cache, v_cache, k_new, v_new, batch, inv_freq, rotary_dim, rope_scale,
                   norm, q_norm_w, k_norm_w, eps, ring, v_norm) -> tuple:
    """attn_rope_qkv's arguments (without the stream), in attn.h's order."""
    n_tok, n_heads, hd = q.shape
    assert q_out.shape == q.shape and q_out.dtype == q.dtype and n_tok >= batch.n_tok
    n_seq_c, n_kv, cap, hd2 = k_cache.shape
    assert hd2 == hd and v_cache.shape == k_cache.shape and n_seq_c >= batch.n_seq
    assert k_new.shape == (n_tok, n_kv, hd) and v_new.shape == k_new.shape
    assert k_new.dtype == k_cache.dtype == v_cache.dtype == v_new.dtype == q.dtype
    return (_dev(q, "q"), _dev(q_out, "q_out"), n_heads, _dev(k_cache, "k_cache"),
            _dev(v_cache, "v_cache"), _dev(k_new, "k_new"), _dev(v_new, "v_new"), n_kv, cap,
            int(ring), _dtype_code(q), n_tok, hd, batch.n_seq, _dev(batch.cu_seq, "cu_seq", torch.int32),
            _dev(batch.start, "start", torch.int32), batch.max_chunk, batch.max_end,
            _dev(inv_freq, "inv_freq", torch.float32) if rotary_dim else None, rotary_dim,
            rope_scale, norm, _dev(q_norm_w, "q_norm_w", torch.float32),
            _dev(k_norm_w, "k_norm_w", torch.float32), eps, int(v_norm))


def prefill_workspace_bytes(batch: Batch, n_heads: int, n_kv: int, head_dim: int) -> int:
    return int(lib().attn_prefill_workspace_bytes(batch.n_seq, n_heads, n_kv, head_dim,
                                                  batch.n_tok, batch.max_chunk, batch.max_end))


def prefill_chunk(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, batch: Batch,
                  scale: float, out: torch.Tensor, workspace: torch.Tensor | None = None,
                  window: int = 0, ring: bool = False, gate: torch.Tensor | None = None,
                  gate_mode: int = GATE_NONE, next_rope: dict | None = None,
                  pending: PrefillPending | None = None, prev: PrefillPending | None = None):
    """Causal attention of a chunk batch; window > 0 keeps keys p-window+1..p;
    ring=True reads key j from cache row j mod cap; gate/gate_mode gate the
    output rows.  next_rope: rope_qkv's keyword arguments for the next chunk,
    run by this call (attn_prefill_chunk_rope_next).  pending: a record that
    receives this chunk's split merge instead of running it, and prev an
    earlier chunk's record whose merge this call runs
    (attn_prefill_chunk_deferred; see prefill_finish)."""
    n_tok, nh, hd = q.shape
    n_seq_c, n_kv, cap, hd2 = k_cache.shape
    assert hd2 == hd and out.shape == (n_tok, nh, hd) and out.dtype == torch.float32
    assert n_seq_c >= batch.n_seq and n_tok >= batch.n_tok
    ws = _dev(workspace, "workspace") if workspace is not None else None
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    args = (_dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dtype_code(q),
            batch.n_seq, nh, n_kv, hd, cap, int(ring), n_tok, _dev(batch.cu_seq, "cu_seq", torch.int32),
            _dev(batch.start, "start", torch.int32), batch.max_chunk, batch.max_end, scale, window,
            *_gate(gate, gate_mode, n_tok, nh, hd, q.dtype), _dev(out, "out"), ws, wsb)
    nxt = None
    if next_rope is not None:
        nr = dict(next_rope)
        nxt = RopeQkvArgs(*_rope_qkv_args(
            nr["q"], nr["q_out"], nr["k_cache"], nr["v_cache"], nr["k_new"], nr["v_new"], nr["batch"],
            nr["inv_freq"], nr["rotary_dim"], nr.get("rope_scale", 1.0), nr.get("norm", NORM_NONE),
            nr.get("q_norm_w"), nr.get("k_norm_w"), nr.get("eps", 1e-6), nr.get("ring", False),
            nr.get("v_norm", False)))
    if pending is not None:
        _check("attn_prefill_chunk_deferred", lib().attn_prefill_chunk_deferred(
            *args, ctypes.byref(nxt) if nxt is not None else None, ctypes.byref(prev) if prev is not None else None,
            ctypes.byref(pending), _stream()))
        return
    assert prev is None, "prev needs a pending record (attn_prefill_chunk_deferred)"
    if nxt is None:
        _check("attn_prefill_chunk", lib().attn_prefill_chunk(*args, _stream()))
        return
    _check("attn_prefill_chunk_rope_next", lib().attn_prefill_chunk_rope_next(*args, ctypes.byref(nxt), _stream()))


def prefill_finish(pending: PrefillPending):
    """Run the merge a pending record owes, on the current stream."""
    _check("attn_prefill_finish", lib().attn_prefill_finish(ctypes.byref(pending), _stream()))


def decode_workspace_bytes(n_seq: int, n_heads: int, n_kv: int, head_dim: int, max_ctx: int) -> int:
    return int(lib().attn_decode_workspace_bytes(n_seq, n_heads, n_kv, head_dim, max_ctx))


def decode_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, ctx: torch.Tensor,
                   max_ctx: int, scale: float, out: torch.Tensor, probs: torch.Tensor | None = None,
                   window: int = 0, ring: bool = False, gate: torch.Tensor | None = None,
                   gate_mode: int = GATE_NONE):
    """decode() without a workspace: the library's static scratch holds the
    split partials (calls that overlap on one GPU race on it)."""
    n_seq, nh, hd = q.shape
    n_seq_c, n_kv, cap, hd2 = k_cache.shape
    assert hd2 == hd and n_seq_c >= n_seq and out.shape == (n_seq, nh, hd)
    assert ctx.shape == (n_seq,) and ctx.dtype == torch.int32
    ld = 0
    if probs is not None:
        assert probs.dim() == 3 and probs.shape[:2] == (n_seq, nh) and probs.dtype == torch.float32
        ld = probs.shape[2]
    st = lib().attn_decode_noalloc(
        _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dtype_code(q), n_seq,
        nh, n_kv, hd, cap, int(ring), _dev(ctx, "ctx"), max_ctx, scale, window,
        *_gate(gate, gate_mode, n_seq, nh, hd, q.dtype), _dev(out, "out"),
        _dev(probs, "probs"), ld, _stream())
    _check("attn_decode_noalloc", st)


def decode_importance(probs: torch.Tensor, ctx: torch.Tensor, max_ctx: int, imp: torch.Tensor,
                      accumulate: bool = True):
    """imp[b][j] (+)= sum over heads of probs[b][h][j], j < ctx[b]."""
    n_seq, nh, ld = probs.shape
    assert probs.dtype == torch.float32 and imp.dtype == torch.float32
    assert imp.dim() == 2 and imp.shape[0] >= n_seq and ctx.shape == (n_seq,) and ctx.dtype == torch.int32
    st = lib().attn_decode_importance(_dev(probs, "probs"), n_seq, nh, ld, _dev(ctx, "ctx"), max_ctx,
                                      _dev(imp, "imp"), imp.shape[1], 1 if accumulate else 0, _stream())
    _check("attn_decode_importance", st)


def decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, ctx: torch.Tensor,
           max_ctx: int, scale: float, out: torch.Tensor, probs: torch.Tensor | None = None,
           workspace: torch.Tensor | None = None, window: int = 0, ring: bool = False,
           gate: torch.Tensor | None = None, gate_mode: int = GATE_NONE):
    """One-query attention over ctx[b] keys; window > 0 keeps the last window keys;
    ring=True reads key j from cache row j mod cap; gate/gate_mode gate the
    output rows."""
    n_seq, nh, hd = q.shape
    n_seq_c, n_kv, cap, hd2 = k_cache.shape
    assert hd2 == hd and n_seq_c >= n_seq and out.shape == (n_seq, nh, hd)
    assert ctx.shape == (n_seq,) and ctx.dtype == torch.int32
    ld = 0
    if probs is not None:
        assert probs.dim() == 3 and probs.shape[:2] == (n_seq, nh) and probs.dtype == torch.float32
        ld = probs.shape[2]
    ws = _dev(workspace, "workspace") if workspace is not None else None
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib().attn_decode(
        _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dtype_code(q), n_seq,
        nh, n_kv, hd, cap, int(ring), _dev(ctx, "ctx"), max_ctx, scale, window,
        *_gate(gate, gate_mode, n_seq, nh, hd, q.dtype), _dev(out, "out"),
        _dev(probs, "probs"), ld, ws, wsb, _stream())
    _check("attn_decode", st)


# ---------------------------------------------------------------- calibration

def calibrate_mfma(n_workgroups: int, iters: int, out: torch.Tensor, random_operands: bool = True) -> float:
    """Launch the matrix-core loop on the current stream (hashed random or
    small constant operands); returns its FLOP count (n_workgroups * 4 waves
    * iters * 4 products * 32768)."""
    assert out.dtype == torch.float32 and out.numel() >= n_workgroups * 4
    _check("attn_calibrate_mfma", lib().attn_calibrate_mfma(n_workgroups, iters, int(bool(random_operands)),
                                                             _dev(out, "out"), _stream()))
    return float(n_workgroups) * 4 * iters * 4 * 32768


def calibrate_read(src: torch.Tensor, n_workgroups: int, out: torch.Tensor) -> int:
    """Launch the streaming read of src on the current stream; returns its bytes."""
    nbytes = src.numel() * src.element_size() // 16 * 16
    assert out.dtype == torch.int32 and out.numel() >= n_workgroups * 4
    _check("attn_calibrate_read", lib().attn_calibrate_read(_dev(src, "src"), nbytes, n_workgroups,
                                                             _dev(out, "out"), _stream()))
    return nbytes
