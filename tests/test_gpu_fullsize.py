"""Parity at the full workload sizes, in the launch configuration bench.py
times (the same chunk driver and chunk sizes).  The Llama-shaped prefill
(4096 positions) and the decode batch (64 sequences) compare every output
row and every probability row with the oracle; the larger workloads compare
sampled rows the oracle computes one at a time: position 0, rows on both
sides of chunk boundaries, the final row and seeded random rows, every query
head of each.  The K/V cache is also checked in full where that is cheap."""
import numpy as np
import pytest
import torch

import oracle
from chunked_prefill_causal_rope_amd import runner, workloads as wl
from parity_util import (check_bf16_rows, check_probs, gain_of, np64, oracle_decode_row,
                         oracle_rows, oracle_table, say)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def sample_positions(n, chunk, seed, extra=12, window=0):
    rng = np.random.default_rng(seed)
    pos = {0, 1, n - 1, n - 2}
    if window:
        # the first rows whose window no longer reaches key 0
        pos.update({window - 1, window, window + 1, window + 63})
    for c in (chunk, 2 * chunk, (n // chunk // 2) * chunk, (n // chunk - 1) * chunk):
        if 0 < c < n:
            pos.update({c - 1, c})
    pos.update(int(x) for x in rng.integers(0, n, extra))
    return sorted(p for p in pos if 0 <= p < n)


def _bits(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy()


def run_prefill(name):
    w = wl.CONFIGS[name]
    say(f"full-size prefill {name}: {w}")
    d = wl.gen_prefill(w, device=DEV)
    run = runner.ChunkedPrefill(w, d, device=DEV)
    run.run_all()
    torch.cuda.synchronize()
    return w, d, run


def check_sequence(w, d, run, b, seed, label, check_cache=True, every_row=False):
    n = d["lengths"][b]
    positions = list(range(n)) if every_row else sample_positions(n, w.chunk, seed, window=w.window)
    pos, ref = oracle_rows(w, d, b, positions)
    got_all = run.gather("out")
    idx = torch.as_tensor(d["cu_seq"][b] + pos, device=got_all.device)
    got = np64(got_all[idx])
    assert np.all(np.isfinite(np64(got_all[d["cu_seq"][b]:d["cu_seq"][b] + n])))
    gain = gain_of(w, d["gate"][idx], got.shape) if w.gate_mode else None
    check_bf16_rows(got, ref, f"{label} seq {b} ({len(pos)} positions x {w.n_heads} heads)", gain=gain)
    if check_cache:
        # every cache row of the sequence equals the oracle's rounded K and the input V
        f = oracle_table(w)
        t0 = d["cu_seq"][b]
        kn = {} if w.norm_style == wl.NORM_NONE else dict(
            norm_style=w.norm_style, norm_w=d["k_norm_w"].cpu().numpy(), eps=w.norm_eps)
        kref = oracle.finish_heads(np64(d["k"][t0:t0 + n]), np.arange(n), f, w.rd, w.rope_scale,
                                   store=oracle.STORE_BF16, **kn)
        want = torch.from_numpy(kref.transpose(1, 0, 2).copy()).to(torch.bfloat16)
        mism = int((_bits(run.k_cache[b, :, :n]) != want.view(torch.int16).numpy()).sum())
        say(f"  K cache mismatching elements: {mism} of {want.numel()}")
        assert mism <= max(1, want.numel() // 1_000_000)
        assert np.array_equal(_bits(run.v_cache[b, :, :n]),
                              _bits(d["v"][t0:t0 + n].transpose(0, 1)))


def test_c1_llama_prefill_full():
    # every one of the 4096 x 32 output rows against the oracle
    w, d, run = run_prefill("c1_llama_prefill")
    check_sequence(w, d, run, 0, 101, "c1", every_row=True)


def test_c3_qwen_varlen_full():
    w, d, run = run_prefill("c3_qwen_varlen")
    say(f"  prompt lengths {d['lengths']}")
    for b in range(w.n_seq):
        check_sequence(w, d, run, b, 300 + b, "c3", check_cache=(b % 3 == 0))


def test_c4_yarn_128k_full():
    w, d, run = run_prefill("c4_yarn_128k")
    check_sequence(w, d, run, 0, 404, "c4", check_cache=False)
    # cache spot check: rows at chunk boundaries and the last row
    f = oracle_table(w)
    rows = np.array([0, 2047, 2048, 65535, 65536, 131071])
    kref = oracle.finish_heads(np64(d["k"][torch.as_tensor(rows, device=DEV)]), rows, f, w.rd,
                               w.rope_scale, store=oracle.STORE_BF16)
    got = run.k_cache[0][:, torch.as_tensor(rows, device=DEV)].transpose(0, 1)
    want = torch.from_numpy(kref).to(torch.bfloat16)
    assert np.array_equal(_bits(got), want.view(torch.int16).numpy())


def check_decode(name, every_seq=False):
    w = wl.CONFIGS[name]
    say(f"full-size decode: {w}")
    d = wl.gen_decode(w, device=DEV)
    step = runner.DecodeStep(w, d, device=DEV)
    step.probs.fill_(float("nan"))
    step.run()
    torch.cuda.synchronize()
    ctx = d["ctx"]
    order = np.argsort(ctx)
    picks = (list(range(len(ctx))) if every_seq else
             sorted({int(order[0]), int(order[1]), int(order[-1]), int(order[-2]),
                     int(order[len(ctx) // 2]), 7}))
    say(f"  checking sequences {picks} with ctx {[ctx[b] for b in picks]}")
    out = np64(step.out)
    cap = step.cap
    for b in picks:
        c = ctx[b]
        o, P = oracle_decode_row(w, d, b, c)
        check_bf16_rows(out[b], o, f"{name} seq {b} ctx {c}")
        pg = np64(step.probs[b])
        assert np.all(np.isnan(pg[:, c:])), "entries past ctx must stay untouched"
        pg = pg[:, :c]
        if w.window and c > w.window:
            # keys before the window: probability exactly 0
            assert np.all(pg[:, :c - w.window] == 0.0)
        check_probs(pg, P, True, f"{name} seq {b} ctx {c}")
    # all outputs finite, every appended row in place
    assert np.all(np.isfinite(out))
    for b, c in enumerate(ctx):
        row = (c - 1) % cap if w.ring else c - 1
        assert torch.equal(step.v_cache[b, :, row], d["v"][b].to(DEV))


def test_c2_decode_full():
    # every one of the 64 sequences: outputs and probabilities of all heads
    check_decode("c2_decode", every_seq=True)


def test_c2_decode_sw4096_full():
    check_decode("c2_decode_sw4096")


def test_c4_yarn_128k_sw4096_full():
    # sliding window of 4096 keys over the 128K prompt: sampled rows on both
    # sides of chunk boundaries, before and after the window fills
    w, d, run = run_prefill("c4_yarn_128k_sw4096")
    check_sequence(w, d, run, 0, 405, "c4 window", check_cache=False)


def test_c2_decode_sw4096_ring_full():
    check_decode("c2_decode_sw4096_ring")


def test_c4_yarn_128k_sw4096_ring_full():
    # the 128K prompt through a 6144-row ring: sampled rows against the
    # oracle, and every output bit-equal to the run over a full-length cache
    w, d, run = run_prefill("c4_yarn_128k_sw4096_ring")
    assert run.k_cache.shape[2] == 6144
    check_sequence(w, d, run, 0, 406, "c4 ring", check_cache=False)
    got = run.gather("out")
    del run
    torch.cuda.empty_cache()
    lin = runner.ChunkedPrefill(wl.CONFIGS["c4_yarn_128k_sw4096"], dict(d, cap=None), device=DEV)
    lin.run_all()
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int32), lin.gather("out").view(torch.int32))


def test_c3_qwen_varlen_gate_full():
    # the varlen Qwen-style prefill with the Qwen3.5 output gate (sigmoid per element)
    w, d, run = run_prefill("c3_qwen_varlen_gate")
    for b in (0, 3, 7):
        check_sequence(w, d, run, b, 500 + b, "c3 gate", check_cache=False)


def test_c2_verify2_full():
    # two new tokens per sequence of the decode batch through the prefill
    # call (the decode kernels), sampled sequences against the oracle
    from parity_util import oracle_verify_rows
    w = wl.CONFIGS["c2_verify2"]
    say(f"full-size verify: {w}")
    d = wl.gen_decode(w, device=DEV)
    step = runner.VerifyStep(w, d, device=DEV)
    step.run()
    torch.cuda.synchronize()
    ctx = d["ctx"]
    order = np.argsort(ctx)
    picks = sorted({int(order[0]), int(order[-1]), int(order[len(ctx) // 2]), 5})
    out = np64(step.out).reshape(len(ctx), 2, w.n_heads, w.head_dim)
    assert np.all(np.isfinite(out))
    for b in picks:
        check_bf16_rows(out[b], oracle_verify_rows(w, d, b, ctx[b]), f"verify seq {b} ctx {ctx[b]}")
    for b, c in enumerate(ctx):
        assert torch.equal(step.v_cache[b, :, c - 2:c], d["v"][2 * b:2 * b + 2].transpose(0, 1).to(DEV))
