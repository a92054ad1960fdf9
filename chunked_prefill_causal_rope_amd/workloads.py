"""Synthetic workloads: the configuration table and seeded input generators.

This module holds no attention or RoPE arithmetic.  It only draws seeded
random inputs (torch generators) and lays out the chunk schedule, so the HIP
path and the CPU oracle can be fed the very same tensors.

Draw order, per workload, from one generator seeded with ``Workload.seed``:
prompt lengths (or decode context lengths), then Q, K, V (or, for decode, the
K cache, the V cache, then the new token's q, k, v), then the q-norm and
k-norm weights when the workload has qk-norm, then the output gate when it
has one.  Values are N(0, 1) drawn in float32 and cast to the workload dtype;
norm weights are 1 + 0.1 * N(0, 1).
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass

import torch

F32, BF16 = "f32", "bf16"
NORM_NONE, NORM_W, NORM_1PW = 0, 1, 2


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str                 # "f32" or "bf16": inputs, rotated Q and the cache
    n_heads: int
    n_kv: int
    head_dim: int
    seed: int
    base: float = 10000.0
    rotary_dim: int | None = None          # None = head_dim
    yarn: tuple | None = None              # (factor, orig_max_pos, beta_fast, beta_slow)
    rope_scale: float = 1.0
    norm_style: int = NORM_NONE
    norm_eps: float = 1e-6
    window: int = 0                        # 0: full causal; W: the last W keys only
    ring: bool = False                     # cache of `cap` rows, position p in row p mod cap
    gate_mode: int = 0                     # output gate: 0 none, 1 sigmoid, 2 softplus/head, 3 softplus
    v_norm: bool = False                   # V rows RMS-normalised before the cache
    # prefill
    n_seq: int = 1
    prompt_len: int = 0                    # fixed length when len_range is None
    len_range: tuple | None = None         # (lo, hi) inclusive, drawn per sequence
    chunk: int = 0
    # decode (chunk = 1 at position ctx-1; new_tokens > 1: that many tokens at
    # ctx-new_tokens .. ctx-1 through the prefill call, e.g. a 2-token verify)
    decode: bool = False
    new_tokens: int = 1
    ctx_range: tuple | None = None         # (lo, hi) inclusive
    cap: int | None = None
    want_probs: bool = False

    @property
    def rd(self) -> int:
        return min(self.rotary_dim or self.head_dim, self.head_dim)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == F32 else torch.bfloat16

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# Five workloads: small f32 correctness case; Llama-style GQA prefill; batched
# decode with probabilities; Qwen-style partial rotary + qk-norm varlen
# prefill; 128K-token YaRN prefill.
CONFIGS = {
    "c0_f32_small": Workload(
        name="c0_f32_small", dtype=F32, n_heads=4, n_kv=2, head_dim=64, seed=1000,
        base=10000.0, prompt_len=64, chunk=16, want_probs=True),
    "c1_llama_prefill": Workload(
        name="c1_llama_prefill", dtype=BF16, n_heads=32, n_kv=8, head_dim=128, seed=1001,
        base=10000.0, prompt_len=4096, chunk=128),
    "c2_decode": Workload(
        name="c2_decode", dtype=BF16, n_heads=32, n_kv=8, head_dim=128, seed=1002,
        base=10000.0, n_seq=64, decode=True, ctx_range=(1024, 32768), cap=32768,
        want_probs=True),
    "c3_qwen_varlen": Workload(
        name="c3_qwen_varlen", dtype=BF16, n_heads=40, n_kv=8, head_dim=128, seed=1003,
        base=1e6, rotary_dim=64, norm_style=NORM_W, norm_eps=1e-6, n_seq=8,
        len_range=(512, 8192), chunk=256, cap=8192),
    "c4_yarn_128k": Workload(
        name="c4_yarn_128k", dtype=BF16, n_heads=64, n_kv=8, head_dim=128, seed=1004,
        base=1e6, yarn=(4.0, 32768, 32.0, 1.0), rope_scale=0.1 * math.log(4.0) + 1.0,
        prompt_len=131072, chunk=2048),
}
# Sliding-window variants (keys p-W+1..p, W = 4096) of the long prefill and
# of the decode batch.
CONFIGS["c4_yarn_128k_sw4096"] = CONFIGS["c4_yarn_128k"].replace(name="c4_yarn_128k_sw4096",
                                                                 window=4096)
CONFIGS["c2_decode_sw4096"] = CONFIGS["c2_decode"].replace(name="c2_decode_sw4096", window=4096)
# The Qwen-style varlen prefill with the Qwen3.5 output gate (sigmoid per
# element).
CONFIGS["c3_qwen_varlen_gate"] = CONFIGS["c3_qwen_varlen"].replace(name="c3_qwen_varlen_gate",
                                                                   gate_mode=1)
# A two-token speculative verify over the decode batch: each sequence adds
# the tokens at ctx-2 and ctx-1 through the prefill call (chunk = 2).
CONFIGS["c2_verify2"] = CONFIGS["c2_decode"].replace(name="c2_verify2", new_tokens=2,
                                                     want_probs=False)
# The same windows over a ring cache: 4096 + 2048 - 1 rows rounded up to a
# multiple of 64 for the prefill (a chunk is written before it attends), 4096
# rows for decode.
CONFIGS["c4_yarn_128k_sw4096_ring"] = CONFIGS["c4_yarn_128k_sw4096"].replace(
    name="c4_yarn_128k_sw4096_ring", ring=True, cap=6144)
CONFIGS["c2_decode_sw4096_ring"] = CONFIGS["c2_decode_sw4096"].replace(
    name="c2_decode_sw4096_ring", ring=True, cap=4096)


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _normal(shape, g, device, dtype):
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(dtype)


def _gate(w: Workload, rows: int, g, device):
    """Output gate values: [rows][n_heads][head_dim], or [rows][n_heads] per head."""
    if not w.gate_mode:
        return None
    shape = (rows, w.n_heads) if w.gate_mode == 2 else (rows, w.n_heads, w.head_dim)
    return _normal(shape, g, device, w.torch_dtype)


def prompt_lengths(w: Workload, g=None, device="cpu") -> list[int]:
    if w.len_range is None:
        return [w.prompt_len] * w.n_seq
    g = g if g is not None else _gen(w.seed, device)
    lo, hi = w.len_range
    return [int(x) for x in torch.randint(lo, hi + 1, (w.n_seq,), generator=g, device=device)]


def gen_prefill(w: Workload, device="cpu"):
    """Packed varlen prefill inputs: q [T][nh][hd], k/v [T][nkv][hd] with the
    sequences concatenated (cu_seq offsets), plus norm weights."""
    g = _gen(w.seed, device)
    lengths = prompt_lengths(w, g, device)
    T = sum(lengths)
    dt = w.torch_dtype
    q = _normal((T, w.n_heads, w.head_dim), g, device, dt)
    k = _normal((T, w.n_kv, w.head_dim), g, device, dt)
    v = _normal((T, w.n_kv, w.head_dim), g, device, dt)
    qw = kw = None
    if w.norm_style != NORM_NONE:
        qw = (1.0 + 0.1 * torch.randn((w.head_dim,), generator=g, device=device)).float()
        kw = (1.0 + 0.1 * torch.randn((w.head_dim,), generator=g, device=device)).float()
    cu = [0]
    for n in lengths:
        cu.append(cu[-1] + n)
    cap = w.cap if w.cap is not None else max(lengths)
    gate = _gate(w, T, g, device)
    return dict(q=q, k=k, v=v, lengths=lengths, cu_seq=cu, q_norm_w=qw, k_norm_w=kw, cap=cap,
                gate=gate)


def gen_decode(w: Workload, device="cpu"):
    """Decode inputs: ctx[b] counts the new tokens, the cache holds the
    ctx[b]-new_tokens prior rows (already rotated; every cache row is drawn;
    with a ring, row r holds the latest position congruent to r), and the new
    tokens' q/k/v ([n_seq * new_tokens] rows, sequence-major) sit at
    positions ctx[b]-new_tokens .. ctx[b]-1."""
    g = _gen(w.seed, device)
    lo, hi = w.ctx_range
    ctx = [int(x) for x in torch.randint(lo, hi + 1, (w.n_seq,), generator=g, device=device)]
    cap = w.cap if w.cap is not None else max(ctx)
    dt = w.torch_dtype
    kc = _normal((w.n_seq, w.n_kv, cap, w.head_dim), g, device, dt)
    vc = _normal((w.n_seq, w.n_kv, cap, w.head_dim), g, device, dt)
    n = w.n_seq * w.new_tokens
    q = _normal((n, w.n_heads, w.head_dim), g, device, dt)
    k = _normal((n, w.n_kv, w.head_dim), g, device, dt)
    v = _normal((n, w.n_kv, w.head_dim), g, device, dt)
    qw = kw = None
    if w.norm_style != NORM_NONE:
        qw = (1.0 + 0.1 * torch.randn((w.head_dim,), generator=g, device=device)).float()
        kw = (1.0 + 0.1 * torch.randn((w.head_dim,), generator=g, device=device)).float()
    gate = _gate(w, n, g, device)
    return dict(ctx=ctx, k_cache=kc, v_cache=vc, q=q, k=k, v=v, q_norm_w=qw, k_norm_w=kw,
                cap=cap, gate=gate)


def chunk_schedule(lengths: list[int], chunk: int) -> list[list[tuple[int, int, int]]]:
    """Steps of a varlen chunked prefill: each step takes the next <= chunk
    tokens of every unfinished prompt.  Each step is a list of
    (seq, first_position, n_tokens) for the sequences it advances."""
    steps = []
    done = [0] * len(lengths)
    while any(d < n for d, n in zip(done, lengths)):
        step = []
        for b, n in enumerate(lengths):
            if done[b] < n:
                c = min(chunk, n - done[b])
                step.append((b, done[b], c))
                done[b] += c
        steps.append(step)
    return steps


def keys_read(start: int, n: int, window: int = 0) -> int:
    """Unmasked (row, key) pairs of rows at positions start..start+n-1: row p
    reads p+1 keys, or min(p+1, window) with a window."""
    end = start + n
    lo = end if window <= 0 else min(max(window, start), end)   # rows >= lo read `window` keys
    return (lo * (lo + 1) - start * (start + 1)) // 2 + (end - lo) * max(window, 0)


def prefill_flops(w: Workload, lengths: list[int]) -> float:
    """Algorithmic causal attention FLOPs: 4*hd per (row, head, unmasked key);
    row p has p+1 keys (min(p+1, window) with a window)."""
    return float(sum(4 * w.head_dim * w.n_heads * keys_read(0, n, w.window) for n in lengths))
