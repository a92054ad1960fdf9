"""Prefill, then decode on the same cache: a varlen batch of bf16 prompts is
prefilled in chunks through attn_rope_qkv + attn_prefill_chunk, then every
sequence continues with decode steps (attn_rope_qkv of one token, then
attn_decode with probabilities) on the cache the prefill left.  Every prefill
output row and every decode output and probability row is compared with the
oracle's one-shot run of the whole sequence, one token at a time.

needle-core 0.3.1 src/v2/batch.rs: fn prefill_batch (after a batched prefill
the state equals that of feeding the same tokens one at a time, which is what
lets decode steps pick up from it) and the module docs (a multi-turn session
depends on the K/V handed from one chunk to the next)."""
import numpy as np
import pytest
import torch

import oracle
from chunked_prefill_causal_rope_amd import api, runner, workloads as wl
from parity_util import check_bf16_rows, check_probs, np64, oracle_table, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("nh,nkv,chunk,window", [(32, 8, 128, 0), (16, 2, 96, 0), (32, 8, 128, 300)])
def test_prefill_then_decode_matches_one_shot_run(nh, nkv, chunk, window):
    hd, n_dec = 128, 6
    prompts = [700, 1031]
    full = [n + n_dec for n in prompts]
    w = wl.Workload(name="resume", dtype=wl.BF16, n_heads=nh, n_kv=nkv, head_dim=hd, seed=88 + nh + chunk,
                    n_seq=len(prompts), chunk=chunk, window=window)
    say(f"resume: heads {nh}/{nkv} chunk {chunk} window {window} prompts {prompts} + {n_dec} decode steps")
    # the whole sequences' inputs (prompt, then the decoded tokens), seeded
    g = torch.Generator().manual_seed(w.seed)
    q_all = [torch.randn((n, nh, hd), generator=g).to(torch.bfloat16) for n in full]
    k_all = [torch.randn((n, nkv, hd), generator=g).to(torch.bfloat16) for n in full]
    v_all = [torch.randn((n, nkv, hd), generator=g).to(torch.bfloat16) for n in full]
    cap = max(full)
    cu = [0]
    for n in prompts:
        cu.append(cu[-1] + n)
    d = dict(q=torch.cat([q[:n] for q, n in zip(q_all, prompts)]).to(DEV),
             k=torch.cat([k[:n] for k, n in zip(k_all, prompts)]).to(DEV),
             v=torch.cat([v[:n] for v, n in zip(v_all, prompts)]).to(DEV),
             lengths=prompts, cu_seq=cu, cap=cap, q_norm_w=None, k_norm_w=None, gate=None)
    run = runner.ChunkedPrefill(w, d, device=DEV, cap=cap)
    run.run_all()
    pre = run.gather("out")
    # decode steps on the cache the prefill left
    n_seq = len(prompts)
    inv_freq = run.inv_freq
    dec_out, dec_probs = [], []
    wsb = api.decode_workspace_bytes(n_seq, nh, nkv, hd, cap)
    ws = torch.empty(wsb // 4 + 1, dtype=torch.float32, device=DEV)
    for i in range(n_dec):
        pos = [n + i for n in prompts]
        batch = api.Batch(pos, [1] * n_seq, device=DEV)
        q = torch.stack([q_all[b][pos[b]] for b in range(n_seq)]).to(DEV)
        k = torch.stack([k_all[b][pos[b]] for b in range(n_seq)]).to(DEV)
        v = torch.stack([v_all[b][pos[b]] for b in range(n_seq)]).to(DEV)
        q_rot = torch.empty_like(q)
        api.rope_qkv(q, q_rot, run.k_cache, run.v_cache, k, v, batch, inv_freq, w.rd)
        ctx = torch.tensor([p + 1 for p in pos], dtype=torch.int32, device=DEV)
        out = torch.empty((n_seq, nh, hd), dtype=torch.float32, device=DEV)
        probs = torch.full((n_seq, nh, cap), float("nan"), dtype=torch.float32, device=DEV)
        api.decode(q_rot, run.k_cache, run.v_cache, ctx, max(pos) + 1, w.scale, out, probs, ws, window=window)
        dec_out.append(out)
        dec_probs.append(probs)
    torch.cuda.synchronize()

    f = oracle_table(w)
    for b in range(n_seq):
        n, nf = prompts[b], full[b]
        ref = oracle.prefill_sequence(np64(q_all[b]), np64(k_all[b]), np64(v_all[b]), 1, f, w.rd,
                                      w.scale, oracle.STORE_BF16, want_probs=True, window=window)
        got_pre = np64(pre[cu[b]:cu[b] + n])
        check_bf16_rows(got_pre, ref["out"][:n], f"seq {b}: {n} prefill rows")
        for i in range(n_dec):
            p = n + i
            check_bf16_rows(np64(dec_out[i][b]), ref["out"][p], f"seq {b}: decode step {i} (position {p})")
            pg = np64(dec_probs[i][b])
            assert np.all(np.isnan(pg[:, p + 1:])), "entries past ctx must stay untouched"
            check_probs(pg[:, :p + 1], ref["probs"][p][:, :p + 1], True, f"seq {b} step {i}")
        # the cache after the last step: K rows equal the oracle's correctly
        # rounded values (at most one element in 10^6 may sit within ~1e-16
        # of a rounding boundary), V rows are bit copies
        kref = torch.from_numpy(ref["k_cache"]).to(torch.bfloat16)
        mism = int((run.k_cache[b, :, :nf].cpu().view(torch.int16) != kref.view(torch.int16)).sum())
        assert mism <= max(1, kref.numel() // 1_000_000), mism
        assert torch.equal(run.v_cache[b, :, :nf].cpu(), v_all[b].transpose(0, 1))
