"""CPU oracle for causal grouped-query attention with RoPE over a head-major
KV cache.

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package; the product path
never does.  The arithmetic lives in ``oracle.c`` (plain C, double precision,
straight loops); this module only marshals numpy arrays and strings the steps
of a chunked prefill together in the order the pages give.

Sources (page title, then the item on it):
  [ATT] cortiq-engine 0.5.39, src/attention.rs
  [NDL] needle-core 0.3.1, src/v2/batch.rs

Every function here is pinned by ``tests/test_oracle_pins.py`` (worked
examples, closed forms, invariants, a brute-force matrix softmax and a library
attention routine); none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

NORM_NONE, NORM_W, NORM_1PW = 0, 1, 2
STORE_F32, STORE_BF16 = 0, 1

_dp = ctypes.POINTER(ctypes.c_double)
_fp = ctypes.POINTER(ctypes.c_float)
_ip = ctypes.POINTER(ctypes.c_int64)


def build() -> str:
    """Compile oracle.c with gcc (no fast-math, no FMA contraction)."""
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
           "-shared", _SRC, "-o", _LIB_PATH, "-lm", "-lpthread"]
    subprocess.check_call(cmd)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.orc_rope_inv_freq.argtypes = [ctypes.c_int, ctypes.c_double, _fp]
    lib.orc_rope_inv_freq.restype = None
    lib.orc_yarn_inv_freq.argtypes = [ctypes.c_int, ctypes.c_double, ctypes.c_double, ctypes.c_int,
                                      ctypes.c_double, ctypes.c_double, _fp,
                                      ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int)]
    lib.orc_yarn_inv_freq.restype = None
    lib.orc_round_bf16.argtypes = [ctypes.c_double]
    lib.orc_round_bf16.restype = ctypes.c_double
    lib.orc_round_array.argtypes = [_dp, ctypes.c_long, ctypes.c_int]
    lib.orc_round_array.restype = None
    lib.orc_finish_heads.argtypes = [_dp, ctypes.c_int, ctypes.c_int, ctypes.c_int, _ip, _fp,
                                     ctypes.c_int, ctypes.c_double, ctypes.c_int, _fp,
                                     ctypes.c_double, ctypes.c_int, ctypes.c_int]
    lib.orc_finish_heads.restype = None
    lib.orc_attend.argtypes = [_dp, _dp, _dp, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                               ctypes.c_int, ctypes.c_long, _ip, ctypes.c_double, _dp, _dp,
                               ctypes.c_long, ctypes.c_int]
    lib.orc_attend.restype = ctypes.c_int
    lib.orc_attend_window.argtypes = [_dp, _dp, _dp, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int, ctypes.c_long, _ip, ctypes.c_double, _dp, _dp,
                                      ctypes.c_long, ctypes.c_long, ctypes.c_int]
    lib.orc_attend_window.restype = ctypes.c_int
    lib.orc_head_importance.argtypes = [_dp, ctypes.c_int, ctypes.c_long, ctypes.c_long, _dp]
    lib.orc_head_importance.restype = ctypes.c_int
    lib.orc_vnorm_heads.argtypes = [_dp, ctypes.c_long, ctypes.c_int, ctypes.c_double, ctypes.c_int]
    lib.orc_vnorm_heads.restype = None
    lib.orc_output_gate.argtypes = [_dp, _dp, ctypes.c_long, ctypes.c_int, ctypes.c_long, ctypes.c_int]
    lib.orc_output_gate.restype = ctypes.c_int
    _lib = lib
    return lib


def default_threads() -> int:
    env = os.environ.get("OMP_NUM_THREADS")
    n = os.cpu_count() or 1
    if env and env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, min(n, 16))


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


# --------------------------------------------------------------------------
# Tables  ([ATT] fn rope_inv_freq, fn yarn_inv_freq)
# --------------------------------------------------------------------------

def rope_inv_freq(rotary_dim: int, base: float) -> np.ndarray:
    out = np.zeros(rotary_dim // 2, dtype=np.float32)
    _load().orc_rope_inv_freq(rotary_dim, base, out.ctypes.data_as(_fp))
    return out


def yarn_inv_freq(rotary_dim: int, base: float, factor: float, orig_max_pos: int,
                  beta_fast: float, beta_slow: float, return_bounds: bool = False):
    out = np.zeros(rotary_dim // 2, dtype=np.float32)
    lo, hi = ctypes.c_int(0), ctypes.c_int(0)
    _load().orc_yarn_inv_freq(rotary_dim, base, factor, orig_max_pos, beta_fast, beta_slow,
                              out.ctypes.data_as(_fp), ctypes.byref(lo), ctypes.byref(hi))
    if return_bounds:
        return out, lo.value, hi.value
    return out


# --------------------------------------------------------------------------
# Rounding and per-head finish
# --------------------------------------------------------------------------

def round_store(x, store: int) -> np.ndarray:
    """Round every element to the stored dtype (ties to even)."""
    a = _f64(x).copy()
    _load().orc_round_array(a.ctypes.data_as(_dp), a.size, store)
    return a


def finish_heads(x, pos, inv_freq, rotary_dim: int, rope_scale: float = 1.0,
                 norm_style: int = NORM_NONE, norm_w=None, eps: float = 1e-6,
                 store: int = STORE_F32, n_threads: int | None = None) -> np.ndarray:
    """Optional per-head RMS norm, then RoPE, then storage rounding.
    x: [n_tok][n_heads][hd]; pos: [n_tok] absolute positions.  Returns a new
    array.  [ATT] fn finish_projection."""
    a = _f64(x).copy()
    n_tok, n_heads, hd = a.shape
    p = np.ascontiguousarray(np.asarray(pos, dtype=np.int64))
    assert p.shape == (n_tok,)
    f = np.ascontiguousarray(np.asarray(inv_freq, dtype=np.float32))
    rd = min(rotary_dim, hd)
    assert f.shape[0] >= rd // 2
    if norm_style != NORM_NONE:
        w = np.ascontiguousarray(np.asarray(norm_w, dtype=np.float32))
        assert w.shape == (hd,)
        wp = w.ctypes.data_as(_fp)
    else:
        wp = None
    _load().orc_finish_heads(a.ctypes.data_as(_dp), n_tok, n_heads, hd, p.ctypes.data_as(_ip),
                             f.ctypes.data_as(_fp), rd, rope_scale, norm_style, wp, eps, store,
                             n_threads or default_threads())
    return a


GATE_NONE, GATE_SIGMOID, GATE_SOFTPLUS_HEAD, GATE_SOFTPLUS = 0, 1, 2, 3


def vnorm_heads(v, eps: float = 1e-6, store: int = STORE_F32) -> np.ndarray:
    """Scale-less RMS norm of every V head row, v [..][hd]: v / sqrt(mean v^2
    + eps), then the storage rounding.  [ATT] fn vnorm_head."""
    a = _f64(v).copy()
    hd = a.shape[-1]
    _load().orc_vnorm_heads(a.ctypes.data_as(_dp), a.size // hd, hd, eps, store)
    return a


def output_gate(out, gate, mode: int) -> np.ndarray:
    """Gate the attention output out [n][nh][hd] (a new array): mode 1
    multiplies by sigmoid(gate) elementwise, gate [n][nh][hd] ([ATT] fn
    apply_gate); mode 2 by softplus of one value per head, gate [n][nh];
    mode 3 by softplus elementwise ([ATT] fn apply_projected_gate)."""
    o = _f64(out).copy()
    hd = o.shape[-1]
    rows = o.size // hd
    g = _f64(gate).reshape(rows, -1).copy()
    if mode == GATE_NONE:
        return o
    if _load().orc_output_gate(o.ctypes.data_as(_dp), g.ctypes.data_as(_dp), rows, hd,
                               g.shape[1], mode) != 0:
        raise ValueError("oracle output_gate: bad mode")
    return o


# --------------------------------------------------------------------------
# Attention
# --------------------------------------------------------------------------

def attend(q, k_cache, v_cache, qpos, scale: float, want_probs: bool = False,
           n_threads: int | None = None, window: int = 0):
    """q [n_tok][nh][hd]; k_cache, v_cache [nkv][cap][hd] of one sequence;
    row t attends keys 0..qpos[t] -- or, with window > 0, the last `window`
    of them ([ATT] QwenAttnCfg.window; zero probability before).  Returns
    (out [n_tok][nh][hd], probs) where probs is a list-of-rows array
    [n_tok][nh][max(qpos)+1] (zero past each row's length) or None."""
    qa, ka, va = _f64(q), _f64(k_cache), _f64(v_cache)
    n_tok, nh, hd = qa.shape
    nkv, cap, hd2 = ka.shape
    assert hd2 == hd and va.shape == ka.shape and nh % nkv == 0
    qp = np.ascontiguousarray(np.asarray(qpos, dtype=np.int64))
    assert qp.shape == (n_tok,)
    out = np.zeros((n_tok, nh, hd), dtype=np.float64)
    ld = int(qp.max()) + 1 if n_tok else 1
    probs = np.zeros((n_tok, nh, ld), dtype=np.float64) if want_probs else None
    rc = _load().orc_attend_window(qa.ctypes.data_as(_dp), ka.ctypes.data_as(_dp),
                                   va.ctypes.data_as(_dp), n_tok, nh, nkv, hd, cap,
                                   qp.ctypes.data_as(_ip), scale, out.ctypes.data_as(_dp),
                                   probs.ctypes.data_as(_dp) if probs is not None else None, ld,
                                   int(window), n_threads or default_threads())
    if rc != 0:
        raise ValueError("oracle attend: bad arguments")
    return out, probs


def head_importance(probs, ctx: int) -> np.ndarray:
    """Importance of each of the first ctx positions for one decode step:
    the sum over heads of the probability rows, probs [nh][>= ctx].  [ATT]
    the per-head loop of the decode attention (each head's probabilities are
    added into one vector, the total probability each position receives)."""
    pa = _f64(probs)
    nh, ld = pa.shape
    imp = np.zeros(ctx, dtype=np.float64)
    if _load().orc_head_importance(pa.ctypes.data_as(_dp), nh, ctx, ld, imp.ctypes.data_as(_dp)) != 0:
        raise ValueError("oracle head_importance: bad arguments")
    return imp


def prefill_sequence(q_raw, k_raw, v_raw, chunk: int, inv_freq, rotary_dim: int,
                     scale: float, store: int, cap: int | None = None, start: int = 0,
                     rope_scale: float = 1.0, norm_style: int = NORM_NONE, q_norm_w=None,
                     k_norm_w=None, eps: float = 1e-6, want_probs: bool = False,
                     k_cache=None, v_cache=None, n_threads: int | None = None, window: int = 0):
    """Chunked prefill of one prompt.  For each chunk of `chunk` tokens, the
    chunk's K rows are finished (norm, RoPE, rounding) and written with its V
    rows into the head-major cache at their absolute positions BEFORE any of
    the chunk's positions attends ([NDL] module docs, "What has to stay
    sequential"; [ATT] fn qwen_attention_batch appends every position of the
    chunk, then attends with limit s0+bi+1).  Then each chunk row at position
    p attends keys 0..p.  chunk=1 is the sequential per-token path.

    q_raw [T][nh][hd], k_raw/v_raw [T][nkv][hd] (already in the stored dtype).
    Returns dict(out, q_rot, k_cache, v_cache, probs).  An optional existing
    cache (k_cache/v_cache, [nkv][cap][hd]) continues a previous run from
    `start`; unwritten cache rows are NaN."""
    qr, kr, vr = _f64(q_raw), _f64(k_raw), _f64(v_raw)
    T, nh, hd = qr.shape
    nkv = kr.shape[1]
    if cap is None:
        cap = start + T
    if k_cache is None:
        kc = np.full((nkv, cap, hd), np.nan)
        vc = np.full((nkv, cap, hd), np.nan)
    else:
        kc, vc = _f64(k_cache).copy(), _f64(v_cache).copy()
    out = np.zeros((T, nh, hd))
    q_rot = np.zeros((T, nh, hd))
    probs = np.zeros((T, nh, start + T)) if want_probs else None
    chunk = max(1, int(chunk))
    for c0 in range(0, T, chunk):
        c1 = min(T, c0 + chunk)
        pos = np.arange(start + c0, start + c1, dtype=np.int64)
        qc = finish_heads(qr[c0:c1], pos, inv_freq, rotary_dim, rope_scale, norm_style,
                          q_norm_w, eps, store)
        kcn = finish_heads(kr[c0:c1], pos, inv_freq, rotary_dim, rope_scale, norm_style,
                           k_norm_w, eps, store)
        # write the whole chunk first: cache[g][pos] = K'[pos][g], V[pos][g]
        kc[:, start + c0:start + c1, :] = kcn.transpose(1, 0, 2)
        vc[:, start + c0:start + c1, :] = vr[c0:c1].transpose(1, 0, 2)
        o, pr = attend(qc, kc, vc, pos, scale, want_probs, n_threads, window)
        out[c0:c1] = o
        q_rot[c0:c1] = qc
        if want_probs:
            probs[c0:c1, :, :pr.shape[2]] = pr
    return dict(out=out, q_rot=q_rot, k_cache=kc, v_cache=vc, probs=probs)


def prefill_sequence_ring(q_raw, k_raw, v_raw, chunk: int, inv_freq, rotary_dim: int,
                          scale: float, store: int, ring: int, window: int,
                          interleaved: bool = False, rope_scale: float = 1.0,
                          norm_style: int = NORM_NONE, q_norm_w=None, k_norm_w=None,
                          eps: float = 1e-6, n_threads: int | None = None):
    """Chunked prefill of one prompt over a ring cache of `ring` slots per KV
    head: position p is stored in slot p mod ring, overwriting position
    p - ring ([NDL] the per-chunk loop's note on the KV ring: writing p+1
    overwrites the slot of p+1-window, still inside p's window).  A row at
    position p attends keys lo..p, lo = max(0, p-window+1) (lo = 0 without a
    window), each read from its slot.

    interleaved=True is the pages' order: write position p, then attend it,
    one position at a time, which a ring of `window` slots supports.
    interleaved=False writes the whole chunk first, then attends its rows;
    that reads the same keys only while ring >= window + chunk - 1.

    Returns dict(out, q_rot, k_cache, v_cache) with the ring caches
    [nkv][ring][hd] (never-written slots are NaN)."""
    qr, kr, vr = _f64(q_raw), _f64(k_raw), _f64(v_raw)
    T, nh, hd = qr.shape
    nkv = kr.shape[1]
    kc = np.full((nkv, ring, hd), np.nan)
    vc = np.full((nkv, ring, hd), np.nan)
    out = np.zeros((T, nh, hd))
    q_rot = np.zeros((T, nh, hd))
    chunk = max(1, int(chunk))

    def attend_row(qrow, p):
        lo = max(0, p - window + 1) if window > 0 else 0
        slots = np.arange(lo, p + 1) % ring
        o, _ = attend(qrow[None], kc[:, slots, :].copy(), vc[:, slots, :].copy(),
                      np.array([p - lo]), scale, n_threads=n_threads)
        return o[0]

    def write(i, p, kcn, c0):
        kc[:, p % ring, :] = kcn[i - c0]
        vc[:, p % ring, :] = vr[i]

    for c0 in range(0, T, chunk):
        c1 = min(T, c0 + chunk)
        pos = np.arange(c0, c1, dtype=np.int64)
        qc = finish_heads(qr[c0:c1], pos, inv_freq, rotary_dim, rope_scale, norm_style,
                          q_norm_w, eps, store)
        kcn = finish_heads(kr[c0:c1], pos, inv_freq, rotary_dim, rope_scale, norm_style,
                           k_norm_w, eps, store)
        if interleaved:
            for i in range(c0, c1):
                write(i, i, kcn, c0)
                out[i] = attend_row(qc[i - c0], i)
        else:
            for i in range(c0, c1):
                write(i, i, kcn, c0)
            for i in range(c0, c1):
                out[i] = attend_row(qc[i - c0], i)
        q_rot[c0:c1] = qc
    return dict(out=out, q_rot=q_rot, k_cache=kc, v_cache=vc)
