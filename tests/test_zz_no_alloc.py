"""attn_decode_noalloc (the decode call whose split partials live in the
library's static scratch, for callers that cannot allocate) against
attn_decode with a caller workspace, through the C ABI: two calls in a row,
the second with a smaller batch, outputs and probabilities compared bit for
bit (the scratch holds the full split for both, so the same parts are
formed), plus the oracle on sampled rows of each call.  A call too large for
the scratch is refused before any device call."""
import numpy as np
import pytest
import torch

from chunked_prefill_causal_rope_amd import api, runner, workloads as wl
from parity_util import check_bf16_rows, check_probs, np64, oracle_decode_row, say

DEV = "cuda:0"


def test_noalloc_refuses_a_batch_beyond_the_scratch():
    # 4096 x 32 rows need 4096 * 32 * 272 B > 32 MiB even with one part each;
    # the status comes back before any device pointer is touched
    L = api.lib()
    P = __import__("ctypes").c_void_p(4096)
    st = L.attn_decode_noalloc(P, P, P, 1, 4096, 32, 8, 128, 4096, 0, P, 4096, 0.088, 0, None, 0, 0,
                               P, None, 0, None)
    assert st == -5
    assert L.attn_status_string(-5).decode() != "unknown status"


def _call_both(w, d, label):
    step = runner.DecodeStep(w, d, device=DEV)
    step.probs.fill_(float("nan"))
    step.run()                                   # append + attn_decode (workspace)
    torch.cuda.synchronize()
    ref_out, ref_probs = step.out.clone(), step.probs.clone()
    out = torch.full_like(step.out, float("nan"))
    probs = torch.full_like(step.probs, float("nan"))
    api.decode_noalloc(step.q_rot, step.k_cache, step.v_cache, step.ctx, step.max_ctx, w.scale, out, probs)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int32), ref_out.view(torch.int32)), f"{label}: outputs differ"
    same = (probs.view(torch.int32) == ref_probs.view(torch.int32)) | (torch.isnan(probs) & torch.isnan(ref_probs))
    assert bool(same.all()), f"{label}: probabilities differ"
    say(f"  {label}: noalloc == workspace call bit for bit")
    ctx = d["ctx"]
    order = np.argsort(ctx)
    for b in sorted({int(order[0]), int(order[-1])}):
        o, P = oracle_decode_row(w, d, b, ctx[b])
        check_bf16_rows(np64(out[b]), o, f"{label} seq {b} ctx {ctx[b]}")
        check_probs(np64(probs[b])[:, :ctx[b]], P, True, f"{label} seq {b}")


@pytest.mark.gpu
def test_noalloc_matches_workspace_decode_twice():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    big = wl.CONFIGS["c2_decode"]                 # 64 sequences, ctx up to 32768
    say(f"noalloc call 1: {big.name}")
    _call_both(big, wl.gen_decode(big, device=DEV), "call 1 (64 seqs)")
    small = wl.Workload(name="noalloc_small", dtype=wl.BF16, n_heads=16, n_kv=4, head_dim=128, seed=77,
                        n_seq=5, decode=True, ctx_range=(1, 3000), cap=3072, want_probs=True)
    say("noalloc call 2: 5 sequences, 16/4 heads")
    _call_both(small, wl.gen_decode(small, device=DEV), "call 2 (5 seqs)")
