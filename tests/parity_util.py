"""Helpers for the GPU parity tests: oracle references for runner outputs and
the tolerance checks.  Imports the oracle (test infrastructure) and the
product package side by side; no value flows from the GPU into the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from chunked_prefill_causal_rope_amd import workloads as wl

# bf16: per output row (position, head), max_d |dO| <= 2e-2 * RMS_d(O_ref).
BF16_ROW_TOL = 2e-2
# f32: max abs error
F32_ABS_TOL = 1e-4


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def store_of(w: wl.Workload) -> int:
    return oracle.STORE_F32 if w.dtype == wl.F32 else oracle.STORE_BF16


def oracle_table(w: wl.Workload) -> np.ndarray:
    if w.yarn is not None:
        return oracle.yarn_inv_freq(w.rd, w.base, *w.yarn)
    return oracle.rope_inv_freq(w.rd, w.base)


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def norm_kwargs(w, d, which):
    if w.norm_style == wl.NORM_NONE:
        return dict(norm_style=oracle.NORM_NONE)
    return dict(norm_style=w.norm_style, norm_w=d[which].cpu().numpy(), eps=w.norm_eps)


def v_rows(w, v):
    """The V rows the cache should hold: the inputs, or their V-norm."""
    v = np64(v)
    return oracle.vnorm_heads(v, w.norm_eps, store_of(w)) if w.v_norm else v


def gain_of(w, gate, shape):
    """The output gate's factors (f64, from the same gate values), shaped like
    an output of `shape`, or None without a gate."""
    if not w.gate_mode:
        return None
    return oracle.output_gate(np.ones(shape), np64(gate).reshape(shape[:-1] + (-1,)), w.gate_mode)


def gated(w, out, gate):
    """The oracle output after the workload's output gate (if any)."""
    if not w.gate_mode:
        return out
    return oracle.output_gate(out, np64(gate), w.gate_mode)


def oracle_prefill_packed(w, d, chunk, want_probs=False):
    """Oracle chunked prefill of every sequence of a packed batch; returns
    out [T][nh][hd] in packed order plus per-sequence caches."""
    f = oracle_table(w)
    outs, caches, qrots, probs = [], [], [], []
    cu = d["cu_seq"]
    for b, n in enumerate(d["lengths"]):
        sl = slice(cu[b], cu[b] + n)
        qn = norm_kwargs(w, d, "q_norm_w")
        kn = norm_kwargs(w, d, "k_norm_w")
        v_in = v_rows(w, d["v"][sl])
        if w.ring:
            r = oracle.prefill_sequence_ring(
                np64(d["q"][sl]), np64(d["k"][sl]), v_in, chunk, f, w.rd, w.scale,
                store_of(w), ring=d["cap"], window=w.window, rope_scale=w.rope_scale,
                norm_style=qn.get("norm_style", 0), q_norm_w=qn.get("norm_w"),
                k_norm_w=kn.get("norm_w"), eps=w.norm_eps)
            probs.append(None)
        else:
            r = oracle.prefill_sequence(
                np64(d["q"][sl]), np64(d["k"][sl]), v_in, chunk, f, w.rd, w.scale,
                store_of(w), rope_scale=w.rope_scale,
                norm_style=qn.get("norm_style", 0), q_norm_w=qn.get("norm_w"),
                k_norm_w=kn.get("norm_w"), eps=w.norm_eps, want_probs=want_probs, window=w.window)
            probs.append(r["probs"])
        outs.append(gated(w, r["out"], d["gate"][sl] if w.gate_mode else None))
        caches.append((r["k_cache"], r["v_cache"]))
        qrots.append(r["q_rot"])
    return dict(out=np.concatenate(outs), caches=caches, q_rot=np.concatenate(qrots), probs=probs)


def oracle_rows(w, d, b, positions, heads=None):
    """Oracle output of selected rows of sequence b (prompt starting at
    position 0): finish the prefix's keys, finish the selected queries, attend.
    Returns [len(positions)][nh][hd] (all heads)."""
    f = oracle_table(w)
    positions = np.asarray(sorted(positions), dtype=np.int64)
    pmax = int(positions.max())
    t0 = d["cu_seq"][b]
    kn = norm_kwargs(w, d, "k_norm_w")
    qn = norm_kwargs(w, d, "q_norm_w")
    k_raw = np64(d["k"][t0:t0 + pmax + 1])
    v_in = v_rows(w, d["v"][t0:t0 + pmax + 1])
    kc = oracle.finish_heads(k_raw, np.arange(pmax + 1), f, w.rd, w.rope_scale,
                             store=store_of(w), **kn)
    idx = torch.as_tensor(t0 + positions, device=d["q"].device)
    q_raw = np64(d["q"][idx])
    q = oracle.finish_heads(q_raw, positions, f, w.rd, w.rope_scale, store=store_of(w), **qn)
    out, _ = oracle.attend(q, kc.transpose(1, 0, 2).copy(), v_in.transpose(1, 0, 2).copy(),
                           positions, w.scale, window=w.window)
    return positions, gated(w, out, d["gate"][idx] if w.gate_mode else None)


def check_bf16_rows(got: np.ndarray, ref: np.ndarray, label="", gain=None):
    """Per-row criterion; returns (worst row err/rms, tensor-level max/rms, rel rmse).
    gain: an output gate's factors, divided out of both sides first -- the
    bound is on the attention output; a factor per element would otherwise
    scale each element's error and the row RMS differently."""
    if gain is not None:
        got = got / gain
        ref = ref / gain
    got = got.reshape(-1, got.shape[-1])
    ref = ref.reshape(-1, ref.shape[-1])
    assert np.all(np.isfinite(got)), f"{label}: non-finite output"
    rms = np.sqrt(np.mean(ref ** 2, axis=-1))
    err = np.max(np.abs(got - ref), axis=-1)
    worst = float(np.max(err / rms))
    tensor = float(np.max(err) / np.sqrt(np.mean(ref ** 2)))
    rrmse = float(np.sqrt(np.mean((got - ref) ** 2)) / np.sqrt(np.mean(ref ** 2)))
    say(f"  {label}: worst row err/rms {worst:.3e}  tensor max/rms {tensor:.3e}  rel rmse {rrmse:.3e}")
    assert worst <= BF16_ROW_TOL, f"{label}: worst row err/rms {worst}"
    return worst, tensor, rrmse


# bf16 decode probabilities pass through half-precision intermediates: each
# value carries a relative error below 2^-10 (its own rounding and the rounded
# normalising sum's, 2^-11 each) and, below half precision's normal range, an
# absolute error below 2^-24 of its row's largest value.
PROB_REL_TOL = 2.0 ** -10 * 1.01
PROB_ABS_FRAC = 2.0 ** -24


def check_probs(got: np.ndarray, ref: np.ndarray, bf16: bool, label=""):
    """got/ref [rows][n]: each row sums to 1 within 1e-5; bf16: elementwise
    |dP| <= PROB_REL_TOL * P + PROB_ABS_FRAC * max(P_row); f32: max |dP| <=
    1e-4 of the row's RMS."""
    got = got.reshape(-1, got.shape[-1])
    ref = ref.reshape(-1, ref.shape[-1])
    assert np.all(np.isfinite(got)), f"{label}: non-finite probability"
    assert np.allclose(got.sum(-1), 1.0, atol=1e-5), f"{label}: row sums"
    err = np.abs(got - ref)
    if bf16:
        bound = PROB_REL_TOL * ref + PROB_ABS_FRAC * ref.max(-1, keepdims=True)
        worst = float(np.max(err / bound))
        say(f"  {label}: probs worst err/bound {worst:.3f}")
        assert worst <= 1.0, f"{label}: probability error {worst} of the bound"
    else:
        rel = float(np.max(np.max(err, -1) / np.sqrt(np.mean(ref ** 2, -1))))
        say(f"  {label}: probs worst err/rms {rel:.3e}")
        assert rel <= 1e-4, f"{label}: probability error {rel}"


def check_f32(got: np.ndarray, ref: np.ndarray, label=""):
    assert np.all(np.isfinite(got)), f"{label}: non-finite output"
    e = float(np.max(np.abs(got - ref)))
    say(f"  {label}: max abs err {e:.3e}")
    assert e <= F32_ABS_TOL, f"{label}: max abs err {e}"
    return e


def oracle_decode_row(w, d, b, c):
    """Oracle (out [nh][hd], probs [nh][c]) of decode row b with context c:
    the new token's K (finished) and V go to position c-1, the prior rows come
    from the drawn cache (row j mod cap with a ring), keys max(0, c-W)..c-1
    with a window."""
    f = oracle_table(w)
    cap = d["k_cache"].shape[2]
    lo = max(0, c - w.window) if w.window else 0
    pos = np.arange(lo, c)
    rows = torch.as_tensor(pos % cap if w.ring else pos, device=d["k_cache"].device)
    kc = np64(d["k_cache"][b][:, rows]).copy()
    vc = np64(d["v_cache"][b][:, rows]).copy()
    last = np.array([c - 1])
    kc[:, -1] = oracle.finish_heads(np64(d["k"][b:b + 1]), last, f, w.rd, w.rope_scale,
                                    store=store_of(w))[0]
    vc[:, -1] = v_rows(w, d["v"][b])
    q = oracle.finish_heads(np64(d["q"][b:b + 1]), last, f, w.rd, w.rope_scale, store=store_of(w))
    # keys lo..c-1 re-indexed from 0: the row sits at c-1-lo and reads them all
    o, P = oracle.attend(q, kc, vc, np.array([c - 1 - lo]), w.scale, want_probs=True)
    probs = np.zeros((w.n_heads, c))
    probs[:, lo:] = P[0]
    return gated(w, o, d["gate"][b:b + 1] if w.gate_mode else None)[0], probs


def oracle_verify_rows(w, d, b, c):
    """Oracle outputs [n][nh][hd] of the n = w.new_tokens queries of sequence
    b whose context is c: the new tokens' K (finished) and V at positions
    c-n .. c-1, the prior rows from the drawn cache (row j mod cap with a
    ring); query i at position c-n+i attends keys up to itself (the last W
    with a window)."""
    n = w.new_tokens
    f = oracle_table(w)
    cap = d["k_cache"].shape[2]
    first_pos = c - n
    lo = max(0, first_pos - w.window + 1) if w.window else 0
    pos = np.arange(lo, c)
    rows = torch.as_tensor(pos % cap if w.ring else pos, device=d["k_cache"].device)
    kc = np64(d["k_cache"][b][:, rows]).copy()
    vc = np64(d["v_cache"][b][:, rows]).copy()
    new_pos = np.arange(first_pos, c)
    sl = slice(b * n, (b + 1) * n)
    kn = oracle.finish_heads(np64(d["k"][sl]), new_pos, f, w.rd, w.rope_scale, store=store_of(w))
    kc[:, c - n - lo:] = kn.transpose(1, 0, 2)
    vc[:, c - n - lo:] = v_rows(w, d["v"][sl]).transpose(1, 0, 2)
    q = oracle.finish_heads(np64(d["q"][sl]), new_pos, f, w.rd, w.rope_scale, store=store_of(w))
    # keys lo..c-1 re-indexed from 0
    o, _ = oracle.attend(q, kc, vc, new_pos - lo, w.scale, window=w.window)
    return gated(w, o, d["gate"][sl] if w.gate_mode else None)
