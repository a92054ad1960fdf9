"""Host-side drivers for the chunk loop and for a decode step.

Each prefill step issues, through the C ABI and on the current stream:
  attn_rope_apply  (finish the step's query rows into a rotated buffer),
  attn_kv_append   (finish the step's key rows into the cache, copy values),
  attn_prefill_chunk (causal attention of the step's rows over the cache).
That is the order of needle-core 0.3.1 src/v2/batch.rs (prefill_batch walks
the prompt in chunks; a chunk's K/V are written before any of its positions
attends) and of cortiq-engine 0.5.39 src/attention.rs fn qwen_attention_batch.
Varlen batches take, per step, the next <= chunk tokens of every unfinished
prompt; a finished prompt stays in the batch with zero tokens so that batch
index b is always cache slot b.

All inputs are staged per step before any work is timed; the drivers only
launch library calls.
"""
from __future__ import annotations

import torch

from . import api
from .workloads import Workload, chunk_schedule


def tables(w: Workload, device="cuda") -> torch.Tensor:
    """Inverse-frequency table of the workload, computed by the library on the
    host and copied to the device once."""
    if w.yarn is not None:
        f = api.yarn_inv_freq(w.rd, w.base, *w.yarn)
    else:
        f = api.rope_inv_freq(w.rd, w.base)
    return f.to(device)


class ChunkedPrefill:
    def __init__(self, w: Workload, data: dict, device="cuda", chunk: int | None = None,
                 cap: int | None = None, k_cache=None, v_cache=None, start_offset: int = 0):
        self.w = w
        self.device = device
        lengths = data["lengths"]
        cu = data["cu_seq"]
        self.lengths = lengths
        self.cu_seq = cu
        self.chunk = chunk or w.chunk
        n_seq = len(lengths)
        self.cap = cap or data.get("cap") or (start_offset + max(lengths))
        hd, nkv, nh = w.head_dim, w.n_kv, w.n_heads
        dt = w.torch_dtype
        if k_cache is None:
            k_cache = torch.zeros((n_seq, nkv, self.cap, hd), dtype=dt, device=device)
            v_cache = torch.zeros((n_seq, nkv, self.cap, hd), dtype=dt, device=device)
        self.k_cache, self.v_cache = k_cache, v_cache
        self.inv_freq = tables(w, device)
        self.q_norm_w = data["q_norm_w"].to(device) if data.get("q_norm_w") is not None else None
        self.k_norm_w = data["k_norm_w"].to(device) if data.get("k_norm_w") is not None else None
        q, k, v = data["q"], data["k"], data["v"]
        gate = data.get("gate")
        self.steps = []
        for step in chunk_schedule(lengths, self.chunk):
            per_seq = {b: (p, c) for b, p, c in step}
            starts, lens, rows = [], [], []
            for b in range(n_seq):
                p, c = per_seq.get(b, (lengths[b], 0))
                starts.append(start_offset + p)
                lens.append(c)
                rows.extend(range(cu[b] + p, cu[b] + p + c))
            batch = api.Batch(starts, lens, device=device)
            r0, r1 = rows[0], rows[-1] + 1
            if rows == list(range(r0, r1)):
                sl = slice(r0, r1)
                qs, ks, vs = q[sl], k[sl], v[sl]
                gs = gate[sl] if gate is not None else None
            else:
                idx = torch.tensor(rows, dtype=torch.long, device=q.device)
                qs, ks, vs = q[idx], k[idx], v[idx]
                gs = gate[idx] if gate is not None else None
            qs, ks, vs = (x.to(device).contiguous() for x in (qs, ks, vs))
            gs = gs.to(device).contiguous() if gs is not None else None
            n_tok = len(rows)
            self.steps.append(dict(
                batch=batch, rows=rows, q=qs, k=ks, v=vs, gate=gs,
                q_rot=torch.empty_like(qs),
                out=torch.empty((n_tok, nh, hd), dtype=torch.float32, device=device)))
        ws = max(api.prefill_workspace_bytes(s["batch"], nh, nkv, hd) for s in self.steps)
        self.workspace = torch.empty(max(ws, 16) // 4 + 1, dtype=torch.float32, device=device)
        # the deferred loop alternates two: a chunk's partials wait in theirs
        # until the next chunk's launch merges them
        self.workspace_alt = torch.empty_like(self.workspace)

    def rope_kwargs(self, i: int) -> dict:
        """api.rope_qkv's keyword arguments for chunk i."""
        w, s = self.w, self.steps[i]
        return dict(q=s["q"], q_out=s["q_rot"], k_cache=self.k_cache, v_cache=self.v_cache, k_new=s["k"],
                    v_new=s["v"], batch=s["batch"], inv_freq=self.inv_freq, rotary_dim=w.rd,
                    rope_scale=w.rope_scale, norm=w.norm_style, q_norm_w=self.q_norm_w,
                    k_norm_w=self.k_norm_w, eps=w.norm_eps, ring=w.ring, v_norm=w.v_norm)

    def run_step(self, i: int, attend: bool = True, fused: bool = True):
        """One chunk: finish Q and append K/V (one fused call, or the two
        separate calls), then attend."""
        w, s = self.w, self.steps[i]
        if fused:
            api.rope_qkv(**self.rope_kwargs(i))
        else:
            api.rope_apply(s["q"], s["q_rot"], s["batch"], self.inv_freq, w.rd, w.rope_scale,
                           w.norm_style, self.q_norm_w, w.norm_eps)
            api.kv_append(self.k_cache, self.v_cache, s["k"], s["v"], s["batch"], self.inv_freq,
                          w.rd, w.rope_scale, w.norm_style, self.k_norm_w, w.norm_eps, ring=w.ring,
                          v_norm=w.v_norm)
        if attend:
            self.attend_step(i)

    def attend_step(self, i: int, next_rope: dict | None = None, pending=None, prev=None,
                    workspace: torch.Tensor | None = None):
        s = self.steps[i]
        api.prefill_chunk(s["q_rot"], self.k_cache, self.v_cache, s["batch"], self.w.scale,
                          s["out"], self.workspace if workspace is None else workspace,
                          window=self.w.window, ring=self.w.ring, gate=s["gate"],
                          gate_mode=self.w.gate_mode, next_rope=next_rope, pending=pending, prev=prev)

    def run_all(self, fused: bool = True, pipelined: bool = True, deferred: bool = True):
        """The chunk loop.  pipelined: chunk 0's finish, then per chunk one
        call that attends it and finishes the next chunk
        (attn_prefill_chunk_rope_next); deferred (with pipelined): the same
        calls with each split chunk's merge run in the next chunk's launch
        (attn_prefill_chunk_deferred, workspaces alternating, the last merge
        by attn_prefill_finish); otherwise finish + attend per chunk."""
        n = len(self.steps)
        if not (fused and pipelined):
            for i in range(n):
                self.run_step(i, fused=fused)
            return
        api.rope_qkv(**self.rope_kwargs(0))
        if not deferred:
            for i in range(n):
                self.attend_step(i, self.rope_kwargs(i + 1) if i + 1 < n else None)
            return
        recs = (api.PrefillPending(), api.PrefillPending())
        wss = (self.workspace, self.workspace_alt)
        prev = None
        for i in range(n):
            cur = recs[i % 2]
            self.attend_step(i, self.rope_kwargs(i + 1) if i + 1 < n else None, pending=cur, prev=prev,
                             workspace=wss[i % 2])
            prev = cur
        if prev is not None:
            api.prefill_finish(prev)

    def gather(self, key: str) -> torch.Tensor:
        """Per-token results of every step, back in the packed input order."""
        first = self.steps[0][key]
        total = self.cu_seq[-1]
        res = torch.empty((total,) + tuple(first.shape[1:]), dtype=first.dtype, device=first.device)
        for s in self.steps:
            idx = torch.tensor(s["rows"], dtype=torch.long, device=first.device)
            res[idx] = s[key]
        return res


class DecodeStep:
    """One decode step for a batch of sequences: finish the new query, append
    the new key/value at position ctx-1, attend keys 0..ctx-1 (with the
    probabilities when the workload asks for them)."""

    def __init__(self, w: Workload, data: dict, device="cuda", probs_ld_multiple: int = 32):
        self.w = w
        ctx = data["ctx"]
        self.ctx_list = ctx
        self.max_ctx = max(ctx)
        n_seq = len(ctx)
        self.k_cache = data["k_cache"].to(device)
        self.v_cache = data["v_cache"].to(device)
        self.cap = self.k_cache.shape[2]
        self.q = data["q"].to(device).contiguous()
        self.k = data["k"].to(device).contiguous()
        self.v = data["v"].to(device).contiguous()
        self.q_rot = torch.empty_like(self.q)
        self.inv_freq = tables(w, device)
        self.q_norm_w = data["q_norm_w"].to(device) if data.get("q_norm_w") is not None else None
        self.k_norm_w = data["k_norm_w"].to(device) if data.get("k_norm_w") is not None else None
        self.gate = data["gate"].to(device).contiguous() if data.get("gate") is not None else None
        self.batch = api.Batch([c - 1 for c in ctx], [1] * n_seq, device=device)
        self.ctx = torch.tensor(ctx, dtype=torch.int32, device=device)
        self.out = torch.empty((n_seq, w.n_heads, w.head_dim), dtype=torch.float32, device=device)
        # probability rows padded to a multiple of 32 floats by default, so
        # every row starts on a 128-byte line (any probs_ld >= max_ctx works)
        m = max(1, int(probs_ld_multiple))
        probs_ld = (self.max_ctx + m - 1) // m * m
        self.probs = (torch.empty((n_seq, w.n_heads, probs_ld), dtype=torch.float32,
                                  device=device) if w.want_probs else None)
        wsb = api.decode_workspace_bytes(n_seq, w.n_heads, w.n_kv, w.head_dim, self.max_ctx)
        self.workspace = torch.empty(max(wsb, 16) // 4 + 1, dtype=torch.float32, device=device)

    def finish_and_append(self):
        w = self.w
        api.rope_qkv(self.q, self.q_rot, self.k_cache, self.v_cache, self.k, self.v, self.batch,
                     self.inv_freq, w.rd, w.rope_scale, w.norm_style, self.q_norm_w,
                     self.k_norm_w, w.norm_eps, ring=w.ring, v_norm=w.v_norm)

    def attend(self):
        api.decode(self.q_rot, self.k_cache, self.v_cache, self.ctx, self.max_ctx, self.w.scale,
                   self.out, self.probs, self.workspace, window=self.w.window, ring=self.w.ring,
                   gate=self.gate, gate_mode=self.w.gate_mode)

    def run(self):
        self.finish_and_append()
        self.attend()


class VerifyStep:
    """new_tokens (> 1, e.g. a 2-token speculative verify) per sequence of a
    decode batch, through the prefill calls: finish and append the tokens at
    ctx-n .. ctx-1, then attend them (each up to its own position)."""

    def __init__(self, w: Workload, data: dict, device="cuda"):
        self.w = w
        n = w.new_tokens
        ctx = data["ctx"]
        self.ctx_list = ctx
        n_seq = len(ctx)
        self.k_cache = data["k_cache"].to(device)
        self.v_cache = data["v_cache"].to(device)
        self.q = data["q"].to(device).contiguous()
        self.k = data["k"].to(device).contiguous()
        self.v = data["v"].to(device).contiguous()
        self.q_rot = torch.empty_like(self.q)
        self.inv_freq = tables(w, device)
        self.q_norm_w = data["q_norm_w"].to(device) if data.get("q_norm_w") is not None else None
        self.k_norm_w = data["k_norm_w"].to(device) if data.get("k_norm_w") is not None else None
        self.gate = data["gate"].to(device).contiguous() if data.get("gate") is not None else None
        self.batch = api.Batch([c - n for c in ctx], [n] * n_seq, device=device)
        self.out = torch.empty((n_seq * n, w.n_heads, w.head_dim), dtype=torch.float32, device=device)
        wsb = api.prefill_workspace_bytes(self.batch, w.n_heads, w.n_kv, w.head_dim)
        self.workspace = torch.empty(max(wsb, 16) // 4 + 1, dtype=torch.float32, device=device)

    def finish_and_append(self):
        w = self.w
        api.rope_qkv(self.q, self.q_rot, self.k_cache, self.v_cache, self.k, self.v, self.batch,
                     self.inv_freq, w.rd, w.rope_scale, w.norm_style, self.q_norm_w,
                     self.k_norm_w, w.norm_eps, ring=w.ring, v_norm=w.v_norm)

    def attend(self, workspace=None):
        api.prefill_chunk(self.q_rot, self.k_cache, self.v_cache, self.batch, self.w.scale,
                          self.out, self.workspace if workspace is None else workspace,
                          window=self.w.window, ring=self.w.ring, gate=self.gate,
                          gate_mode=self.w.gate_mode)

    def run(self):
        self.finish_and_append()
        self.attend()
