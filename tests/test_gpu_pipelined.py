"""The pipelined chunk loops against the per-chunk loop.  Pipelined: chunk 0's
finish (attn_rope_qkv), then one attn_prefill_chunk_rope_next per chunk that
attends it and finishes the next chunk -- inside the attention launch for
bf16 on the per-token path over an unwrapped cache when the finish needs at
most one workgroup per CU, otherwise as a second launch.  Deferred: the same
loop through attn_prefill_chunk_deferred, where a split chunk's merge runs in
the next chunk's launch (workspaces alternating) and the last one through
attn_prefill_finish.  Per chunk: attn_rope_qkv, then attn_prefill_chunk.
Outputs, rotated queries and both caches must agree bit for bit: the next
chunk's finish writes cache rows past every key the current chunk reads
([NDL] module docs, "What has to stay sequential": a chunk's rows are in the
cache before it attends, which every loop keeps), and the merge is the same
computation wherever it runs."""
import pytest
import torch

from chunked_prefill_causal_rope_amd import api, runner, workloads as wl
from parity_util import say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def _same(a: torch.Tensor, b: torch.Tensor) -> bool:
    ia = a.contiguous().view(torch.int16 if a.element_size() == 2 else torch.int32)
    ib = b.contiguous().view(torch.int16 if b.element_size() == 2 else torch.int32)
    return torch.equal(ia, ib)


CASES = [
    # split calls on the key-split kernel, the RoPE finish in the attention launch
    dict(name="llama_like", dtype=wl.BF16, n_heads=32, n_kv=8, head_dim=128, prompt_len=1000, chunk=128),
    # qk-norm and partial rotary (per-token path), a varlen batch
    dict(name="varlen_qknorm", dtype=wl.BF16, n_heads=10, n_kv=2, head_dim=128, n_seq=3, len_range=(40, 700),
         chunk=64, cap=700, rotary_dim=64, norm_style=wl.NORM_W, base=1e6),
    # a finish too large to ride in the attention launch (its own launch)
    dict(name="varlen_qknorm_wide_chunks", dtype=wl.BF16, n_heads=10, n_kv=2, head_dim=128, n_seq=4,
         len_range=(40, 700), chunk=256, cap=700, rotary_dim=64, norm_style=wl.NORM_W, base=1e6),
    # many sequences: 256-row items on the ping-pong kernel
    dict(name="wide", dtype=wl.BF16, n_heads=32, n_kv=8, head_dim=128, n_seq=32, len_range=(1, 200), chunk=64,
         cap=200),
    dict(name="hd64", dtype=wl.BF16, n_heads=16, n_kv=2, head_dim=64, prompt_len=500, chunk=96),
    # a window, output gates and V-norm ride along unchanged
    dict(name="window_gate_vnorm", dtype=wl.BF16, n_heads=16, n_kv=4, head_dim=128, prompt_len=700, chunk=128,
         window=200, gate_mode=1, v_norm=True, norm_style=wl.NORM_1PW),
    # fallbacks: rotary_dim not a multiple of 8, a wrapped ring, the small-chunk
    # (decode-kernel) path, float32
    dict(name="rotary36", dtype=wl.BF16, n_heads=8, n_kv=2, head_dim=128, prompt_len=300, chunk=64,
         rotary_dim=36),
    dict(name="ring_wrapped", dtype=wl.BF16, n_heads=8, n_kv=2, head_dim=128, prompt_len=600, chunk=64,
         window=128, ring=True, cap=192),
    dict(name="chunk2", dtype=wl.BF16, n_heads=8, n_kv=2, head_dim=128, prompt_len=40, chunk=2),
    dict(name="f32", dtype=wl.F32, n_heads=8, n_kv=2, head_dim=64, prompt_len=200, chunk=64),
]


LOOPS = {"per_chunk": dict(pipelined=False), "pipelined": dict(pipelined=True, deferred=False),
         "deferred": dict(pipelined=True, deferred=True)}


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_pipelined_loops_equal_per_chunk_loop(case):
    kw = dict(case)
    w = wl.Workload(seed=71, **kw)
    say(f"pipelined and deferred vs per-chunk: {w}")
    d = wl.gen_prefill(w, device=DEV)
    runs = {}
    for name, how in LOOPS.items():
        r = runner.ChunkedPrefill(w, d, device=DEV)
        r.run_all(**how)
        runs[name] = r
    torch.cuda.synchronize()
    a = runs["per_chunk"]
    for name in ("pipelined", "deferred"):
        b = runs[name]
        for key in ("out", "q_rot"):
            assert _same(a.gather(key), b.gather(key)), (name, key)
        assert _same(a.k_cache, b.k_cache) and _same(a.v_cache, b.v_cache), name


def _split_step(r):
    w = r.w
    for i, s in enumerate(r.steps):
        if api.prefill_workspace_bytes(s["batch"], w.n_heads, w.n_kv, w.head_dim) > 0:
            return i
    raise AssertionError("no split chunk")


def test_deferred_merge_across_paths():
    """A pending merge runs on its own launch when the next call cannot carry
    it (another head size, float32), and a workspace that overlaps the
    pending partials is refused before anything is launched."""
    wa = wl.Workload(seed=72, name="hd64", dtype=wl.BF16, n_heads=16, n_kv=2, head_dim=64, prompt_len=500,
                     chunk=96)
    wb = wl.Workload(seed=73, name="hd128", dtype=wl.BF16, n_heads=32, n_kv=8, head_dim=128, prompt_len=700,
                     chunk=128)
    wc = wl.Workload(seed=74, name="f32", dtype=wl.F32, n_heads=8, n_kv=2, head_dim=64, prompt_len=200,
                     chunk=64)
    runs = []
    for w in (wa, wb, wc):
        say(f"deferred across paths: {w}")
        r = runner.ChunkedPrefill(w, wl.gen_prefill(w, device=DEV), device=DEV)
        r.run_all(pipelined=False)             # reference outputs, caches filled
        runs.append(r)
    ra, rb, rc = runs
    ia, ib = _split_step(ra), _split_step(rb)
    ic = len(rc.steps) - 1
    refs = [ra.steps[ia]["out"].clone(), rb.steps[ib]["out"].clone(), rc.steps[ic]["out"].clone()]
    for r, i in ((ra, ia), (rb, ib), (rc, ic)):
        r.steps[i]["out"].fill_(float("nan"))
    rec_a, rec_b, rec_c = api.PrefillPending(), api.PrefillPending(), api.PrefillPending()
    ra.attend_step(ia, pending=rec_a)
    assert rec_a.active == 1 and rec_a.head_dim == 64
    # the pending partials sit in ra.workspace: reusing it is refused
    with pytest.raises(api.AttnError) as e:
        ra.attend_step(ia, pending=api.PrefillPending(), prev=rec_a, workspace=ra.workspace)
    assert e.value.status == -1
    # the pending merge writes its chunk's output rows: a call writing the same rows is refused
    with pytest.raises(api.AttnError) as e:
        ra.attend_step(ia, pending=api.PrefillPending(), prev=rec_a, workspace=ra.workspace_alt)
    assert e.value.status == -1
    rb.attend_step(ib, pending=rec_b, prev=rec_a)      # hd 64 merge alone, then hd 128 attention
    assert rec_b.active == 1 and rec_b.head_dim == 128
    rc.attend_step(ic, pending=rec_c, prev=rec_b)      # bf16 merge alone, then the float32 path
    assert rec_c.active == 0
    api.prefill_finish(rec_c)
    torch.cuda.synchronize()
    for r, i, ref in zip((ra, rb, rc), (ia, ib, ic), refs):
        assert _same(r.steps[i]["out"], ref), r.w.name
