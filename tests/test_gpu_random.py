"""Seeded random configurations through the whole path, against the oracle:
dtype, head size, GQA group, partial rotary, qk-norm style, varlen prompts,
chunk size (1 and 2 included: the decode kernels), sliding window, ring
cache, output gate and V-norm are drawn per case, so combinations no
hand-written case covers are exercised.  Each case is small enough for the
oracle to finish in well under a second."""
import numpy as np
import pytest
import torch

from chunked_prefill_causal_rope_amd import runner, workloads as wl
from parity_util import (check_bf16_rows, check_f32, check_probs, gain_of, np64, oracle_decode_row,
                         oracle_prefill_packed, say)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def _draw_prefill(seed):
    rng = np.random.default_rng(seed)
    dtype = wl.BF16 if rng.random() < 0.75 else wl.F32
    hd = int(rng.choice([64, 128]))
    nh, nkv = [(4, 1), (8, 2), (6, 3), (16, 2), (12, 4), (8, 8)][rng.integers(6)]
    rd = int(rng.choice([hd, hd // 2]))
    norm = int(rng.integers(3))
    n_seq = int(rng.integers(1, 5))
    chunk = int(rng.choice([1, 2, 3, 16, 64, 100]))
    hi = 300 if chunk >= 16 else 60
    window = int(rng.choice([0, 0, 1, 17, 64, 200]))
    ring = window > 0 and rng.random() < 0.4
    cap = None
    if ring:
        need = window + chunk - 1
        cap = (need + 63) // 64 * 64 if dtype == wl.BF16 else need + int(rng.integers(3))
    gate = int(rng.integers(4)) if rng.random() < 0.5 else 0
    v_norm = bool(rng.random() < 0.3)
    return wl.Workload(name=f"rand{seed}", dtype=dtype, n_heads=nh, n_kv=nkv, head_dim=hd,
                       seed=seed, base=float(rng.choice([1e4, 1e6])), rotary_dim=rd,
                       norm_style=norm, n_seq=n_seq, len_range=(1, hi), chunk=chunk,
                       window=window, ring=bool(ring), cap=cap, gate_mode=gate, v_norm=v_norm)


@pytest.mark.parametrize("seed", [*range(2000, 2064), *range(5000, 5200)])
def test_random_prefill_configs(seed):
    w = _draw_prefill(seed)
    say(f"random prefill {w}")
    d = wl.gen_prefill(w)
    if w.ring:
        d = dict(d, cap=w.cap)
    run = runner.ChunkedPrefill(w, d, device=DEV)
    run.run_all()
    torch.cuda.synchronize()
    ref = oracle_prefill_packed(w, d, w.chunk)
    got = np64(run.gather("out"))
    if w.dtype == wl.BF16:
        check_bf16_rows(got, ref["out"], w.name, gain=gain_of(w, d["gate"], got.shape))
    else:
        check_f32(got, ref["out"], w.name)


def _draw_decode(seed):
    rng = np.random.default_rng(seed)
    dtype = wl.BF16 if rng.random() < 0.75 else wl.F32
    nh, nkv = [(8, 2), (16, 4), (32, 8), (16, 2), (8, 8)][rng.integers(5)]
    hd = int(rng.choice([64, 128]))
    n_seq = int(rng.integers(1, 7))
    window = int(rng.choice([0, 0, 1, 50, 700]))
    ring = window > 0 and rng.random() < 0.4
    cap = int(rng.integers(window, window + 300)) if ring else 2048
    gate = int(rng.integers(4)) if rng.random() < 0.5 else 0
    return wl.Workload(name=f"rdec{seed}", dtype=dtype, n_heads=nh, n_kv=nkv, head_dim=hd,
                       seed=seed, n_seq=n_seq, decode=True, ctx_range=(1, 2048), cap=cap,
                       want_probs=True, window=window, ring=bool(ring), gate_mode=gate,
                       v_norm=bool(rng.random() < 0.3))


@pytest.mark.parametrize("seed", [*range(3000, 3032), *range(6000, 6100)])
def test_random_decode_configs(seed):
    w = _draw_decode(seed)
    say(f"random decode {w}")
    d = wl.gen_decode(w)
    step = runner.DecodeStep(w, d, device=DEV, probs_ld_multiple=1)
    step.probs.fill_(float("nan"))
    step.run()
    torch.cuda.synchronize()
    got_o = np64(step.out)
    got_p = np64(step.probs)
    for b, c in enumerate(d["ctx"]):
        o, P = oracle_decode_row(w, d, b, c)
        if w.dtype == wl.BF16:
            gain = gain_of(w, d["gate"][b] if w.gate_mode else None, o.shape)
            check_bf16_rows(got_o[b], o, f"{w.name} seq {b} ctx {c}", gain=gain)
        else:
            check_f32(got_o[b], o, f"{w.name} seq {b} ctx {c}")
        assert np.all(np.isnan(got_p[b, :, c:]))
        check_probs(got_p[b, :, :c], P, w.dtype == wl.BF16, f"{w.name} seq {b}")
