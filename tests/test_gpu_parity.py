"""GPU parity: every library entry point against the CPU oracle on the same
seeded inputs.  Bars: bit-exact cache layout (V rows, untouched rows), K and
rotated Q equal to the oracle's correctly rounded values, f32 outputs within
1e-4 absolute, bf16 outputs within 2e-2 of each output row's RMS."""
import numpy as np
import pytest
import torch

import oracle
from chunked_prefill_causal_rope_amd import api, runner, workloads as wl
from parity_util import (PROB_ABS_FRAC, PROB_REL_TOL, check_bf16_rows, check_f32, check_probs, gain_of, np64,
                         oracle_decode_row, oracle_prefill_packed, oracle_table, oracle_verify_rows, say,
                         store_of)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def _bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy()
    return t.view(torch.int32).numpy()


def _to_dtype_bits(x: np.ndarray, dtype) -> np.ndarray:
    return _bits(torch.from_numpy(x).to(dtype))


# ------------------------------------------------------------------ RoPE

@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
@pytest.mark.parametrize("hd,rd,norm,scale", [
    (128, 128, wl.NORM_NONE, 1.0),
    (128, 64, wl.NORM_W, 1.0),
    (64, 64, wl.NORM_1PW, 1.1386294),
    (128, 32, wl.NORM_NONE, 1.1386294),
])
@pytest.mark.parametrize("starts", [(0, 17, 131000), (5, 2**30 - 20, 2**31 - 50)])
def test_rope_apply_matches_oracle(dtype, hd, rd, norm, scale, starts):
    # rope_scale crosses the ABI as a float (the page's f32 field): the oracle
    # gets that same float value.  The second set of starts reaches angles
    # near 2^31 radians (the largest positions an int32 holds).
    scale = float(np.float32(scale))
    say(f"rope_apply dtype={dtype} hd={hd} rd={rd} norm={norm} scale={scale} starts={starts}")
    w = wl.Workload(name="rope", dtype=dtype, n_heads=6, n_kv=2, head_dim=hd, seed=11,
                    rotary_dim=rd, norm_style=norm, rope_scale=scale, base=1e4,
                    n_seq=3, len_range=(1, 40), chunk=40)
    d = wl.gen_prefill(w)
    starts = list(starts)
    batch = api.Batch(starts, d["lengths"], device=DEV)
    x = d["q"].to(DEV)
    y = torch.full_like(x, float("nan"))
    f = runner.tables(w, DEV)
    qw = d["q_norm_w"].to(DEV) if norm else None
    api.rope_apply(x, y, batch, f, rd, scale, norm, qw, w.norm_eps)
    torch.cuda.synchronize()
    pos = np.concatenate([np.arange(s, s + n) for s, n in zip(starts, d["lengths"])])
    kw = dict(norm_style=norm, norm_w=d["q_norm_w"].numpy() if norm else None, eps=w.norm_eps)
    ref = oracle.finish_heads(np64(d["q"]), pos, oracle_table(w), rd, scale, store=store_of(w), **kw)
    diff = _bits(y) != _to_dtype_bits(ref, w.torch_dtype)
    say(f"  mismatching elements: {int(diff.sum())} of {diff.size}")
    # double arithmetic on both sides: the stored values agree bit for bit
    # except where the exact value sits within ~1e-16 of a rounding boundary
    assert diff.sum() <= max(1, diff.size // 100000)
    # in place gives the same bits
    x2 = x.clone()
    api.rope_apply(x2, x2, batch, f, rd, scale, norm, qw, w.norm_eps)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(x2), _bits(y))


# ------------------------------------------------------------------ append

@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
def test_kv_append_layout_and_sentinels(dtype):
    say(f"kv_append layout dtype={dtype}")
    w = wl.Workload(name="app", dtype=dtype, n_heads=8, n_kv=4, head_dim=128, seed=12,
                    rotary_dim=128, base=1e4, n_seq=3, len_range=(5, 70), chunk=70,
                    norm_style=wl.NORM_W)
    d = wl.gen_prefill(w)
    cap = 300
    starts = [0, 100, cap - d["lengths"][2]]
    batch = api.Batch(starts, d["lengths"], device=DEV)
    kc = torch.full((3, w.n_kv, cap, w.head_dim), float("nan"), dtype=w.torch_dtype, device=DEV)
    vc = torch.full_like(kc, float("nan"))
    before_k, before_v = _bits(kc), _bits(vc)
    f = runner.tables(w, DEV)
    api.kv_append(kc, vc, d["k"].to(DEV), d["v"].to(DEV), batch, f, w.rd, 1.0, w.norm_style,
                  d["k_norm_w"].to(DEV), w.norm_eps)
    torch.cuda.synchronize()
    gk, gv = _bits(kc), _bits(vc)
    written = np.zeros(kc.shape[:3], dtype=bool)
    cu = d["cu_seq"]
    mism = 0
    for b, (s, n) in enumerate(zip(starts, d["lengths"])):
        written[b, :, s:s + n] = True
        rows = slice(cu[b], cu[b] + n)
        pos = np.arange(s, s + n)
        ref = oracle.finish_heads(np64(d["k"][rows]), pos, oracle_table(w), w.rd, 1.0,
                                  norm_style=w.norm_style, norm_w=d["k_norm_w"].numpy(),
                                  eps=w.norm_eps, store=store_of(w))
        want_k = _to_dtype_bits(ref.transpose(1, 0, 2).copy(), w.torch_dtype)
        mism += int((gk[b, :, s:s + n] != want_k).sum())
        want_v = _bits(d["v"][rows].transpose(0, 1).contiguous())
        assert np.array_equal(gv[b, :, s:s + n], want_v), "V rows must be a bit copy"
    say(f"  K mismatching elements: {mism}")
    assert mism <= 1
    # every row outside the appended ranges keeps its sentinel bits
    assert np.array_equal(gk[~written], before_k[~written])
    assert np.array_equal(gv[~written], before_v[~written])


@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
@pytest.mark.parametrize("hd,rd,norm,scale,nh,nkv", [
    (128, 128, wl.NORM_NONE, 1.0, 32, 8),        # one launch, 40 heads in 3 passes
    (128, 64, wl.NORM_W, 1.0, 40, 8),            # partial rotary, qk-norm
    (64, 64, wl.NORM_1PW, 1.1386294, 6, 2),
    (128, 30, wl.NORM_W, 1.0, 6, 2),             # rotary_dim not a multiple of 8: two launches
    (128, 128, wl.NORM_NONE, 1.0, 64, 8),        # 72 heads: more than one group of passes
])
def test_rope_qkv_equals_separate_calls(dtype, hd, rd, norm, scale, nh, nkv):
    scale = float(np.float32(scale))
    say(f"rope_qkv dtype={dtype} hd={hd} rd={rd} norm={norm} nh={nh} nkv={nkv}")
    w = wl.Workload(name="qkv", dtype=dtype, n_heads=nh, n_kv=nkv, head_dim=hd, seed=13,
                    rotary_dim=rd, norm_style=norm, rope_scale=scale, base=1e4,
                    n_seq=3, len_range=(1, 40), chunk=40)
    d = wl.gen_prefill(w)
    cap = 200
    starts = [0, 17, cap - d["lengths"][2]]
    batch = api.Batch(starts, d["lengths"], device=DEV)
    f = runner.tables(w, DEV)
    qw = d["q_norm_w"].to(DEV) if norm else None
    kw = d["k_norm_w"].to(DEV) if norm else None
    q, k, v = d["q"].to(DEV), d["k"].to(DEV), d["v"].to(DEV)
    outs = []
    for fused in (False, True):
        y = torch.full_like(q, float("nan"))
        kc = torch.full((3, nkv, cap, hd), float("nan"), dtype=w.torch_dtype, device=DEV)
        vc = torch.full_like(kc, float("nan"))
        if fused:
            api.rope_qkv(q, y, kc, vc, k, v, batch, f, rd, scale, norm, qw, kw, w.norm_eps)
        else:
            api.rope_apply(q, y, batch, f, rd, scale, norm, qw, w.norm_eps)
            api.kv_append(kc, vc, k, v, batch, f, rd, scale, norm, kw, w.norm_eps)
        torch.cuda.synchronize()
        outs.append((_bits(y), _bits(kc), _bits(vc)))
    for a, b in zip(*outs):
        assert np.array_equal(a, b)


def _midpoint_inputs(n_scales: int):
    """Pairs (rope_scale, bf16 inputs x) for which x * rope_scale (exact in
    double) rounds to a float lying exactly halfway between two bfloat16
    neighbours, while the product itself is not that midpoint, and for which
    rounding through float gives a different bfloat16 than rounding once (the
    oracle's).  Found by search over float scales near 1.1386 and every
    finite non-zero bfloat16, subnormals included."""
    bits = np.arange(1 << 16, dtype=np.uint32)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]                # drop inf / NaN
    bits = bits[(bits & 0x7FFF) != 0]                        # drop zeros
    x = (bits << 16).view(np.float32).astype(np.float64)
    x = x[np.abs(x) < 2.0 ** 120]
    found = []
    s = np.float32(1.1386294)
    while len(found) < n_scales:
        s = np.nextafter(s, np.float32(2.0))
        p = x * float(s)
        f = p.astype(np.float32)
        mid = ((f.view(np.uint32) & 0xFFFF) == 0x8000) & (f.astype(np.float64) != p)
        if not mid.any():
            continue
        via_float = torch.from_numpy(f[mid]).to(torch.bfloat16).float().numpy().astype(np.float64)
        once = oracle.round_store(p[mid], oracle.STORE_BF16)
        sel = x[mid][via_float != once]
        if sel.size:
            found.append((float(s), sel))
    return found


@pytest.mark.parametrize("hd,rd", [(128, 128), (128, 64), (64, 64), (128, 36)])
def test_bf16_single_rounding_at_float_midpoints(hd, rd):
    """At position 0 the rotation is the identity, so every rotary output is
    x * rope_scale.  Inputs are chosen so that this product's float image is a
    bfloat16 midpoint: the stored bits must still be the oracle's single
    rounding, for queries and for keys.  (rd = 36 takes the general path.)"""
    cases = _midpoint_inputs(4)
    for scale, xs in cases:
        say(f"midpoints hd={hd} rd={rd} scale={scale!r} n={xs.size}")
        n_seq, nh = 5, 3
        rng = np.random.default_rng(5)
        # every sequence is one token at position 0; the chosen values fill
        # the rotary dims of every head, cycled, the rest random
        vals = rng.standard_normal((n_seq, nh, hd))
        vals[:, :, :rd] = np.resize(xs, n_seq * nh * rd).reshape(n_seq, nh, rd)
        x = torch.from_numpy(vals).to(torch.bfloat16)
        batch = api.Batch([0] * n_seq, [1] * n_seq, device=DEV)
        f = torch.from_numpy(oracle.rope_inv_freq(rd, 1e4)).to(DEV)
        ref = oracle.finish_heads(np64(x), np.zeros(n_seq, np.int64), oracle.rope_inv_freq(rd, 1e4),
                                  rd, scale, store=oracle.STORE_BF16)
        want = _to_dtype_bits(ref, torch.bfloat16)
        y = torch.full_like(x, float("nan"), device=DEV)
        api.rope_apply(x.to(DEV), y, batch, f, rd, scale, 0, None, 1e-6)
        kc = torch.full((n_seq, nh, 1, hd), float("nan"), dtype=torch.bfloat16, device=DEV)
        vc = torch.full_like(kc, float("nan"))
        api.kv_append(kc, vc, x.to(DEV), x.to(DEV), batch, f, rd, scale, 0, None, 1e-6)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(y), want)
        assert np.array_equal(_bits(kc)[:, :, 0, :], want)


# ------------------------------------------------------------------ f32 path

def test_c0_f32_prefill_and_sequential_probs():
    w = wl.CONFIGS["c0_f32_small"]
    say(f"c0 f32 prefill {w}")
    d = wl.gen_prefill(w)
    ref_seq = oracle_prefill_packed(w, d, 1, want_probs=True)
    for chunk in (16, 1, 64, 7):
        run = runner.ChunkedPrefill(w, d, device=DEV, chunk=chunk)
        run.run_all()
        torch.cuda.synchronize()
        check_f32(np64(run.gather("out")), ref_seq["out"], f"chunk {chunk}")
    # per-position probabilities: 64 decode calls, one per position
    f = runner.tables(w, DEV)
    kc = torch.zeros((1, w.n_kv, 64, w.head_dim), dtype=torch.float32, device=DEV)
    vc = torch.zeros_like(kc)
    q = d["q"].to(DEV)
    k = d["k"].to(DEV)
    v = d["v"].to(DEV)
    ws = torch.empty(1 << 16, dtype=torch.float32, device=DEV)
    P_ref = ref_seq["probs"][0]
    worst_p = 0.0
    for p in range(64):
        batch = api.Batch([p], [1], device=DEV)
        qr = torch.empty_like(q[p:p + 1])
        api.rope_apply(q[p:p + 1].contiguous(), qr, batch, f, w.rd)
        api.kv_append(kc, vc, k[p:p + 1].contiguous(), v[p:p + 1].contiguous(), batch, f, w.rd)
        out = torch.empty((1, w.n_heads, w.head_dim), dtype=torch.float32, device=DEV)
        probs = torch.full((1, w.n_heads, 64), float("nan"), device=DEV)
        ctx = torch.tensor([p + 1], dtype=torch.int32, device=DEV)
        api.decode(qr, kc, vc, ctx, p + 1, w.scale, out, probs, ws)
        torch.cuda.synchronize()
        check_f32(np64(out)[0], ref_seq["out"][p], f"decode pos {p}") if p % 16 == 0 else None
        assert float(np.max(np.abs(np64(out)[0] - ref_seq["out"][p]))) <= 1e-4
        pg = np64(probs)[0]
        assert np.all(np.isnan(pg[:, p + 1:])), "entries past ctx must stay untouched"
        dp = np.max(np.abs(pg[:, :p + 1] - P_ref[p, :, :p + 1]))
        worst_p = max(worst_p, float(dp))
        assert np.allclose(pg[:, :p + 1].sum(-1), 1.0, atol=1e-5)
    say(f"  probs max abs err {worst_p:.3e}")
    assert worst_p <= 1e-4


# ------------------------------------------------------------------ bf16 prefill

CASES = [
    # name, nh, nkv, hd, T, chunk
    ("gqa4_hd128", 8, 2, 128, 300, 128),
    ("gqa4_hd128_small_chunks", 8, 2, 128, 200, 16),
    ("mha_hd64", 3, 3, 64, 190, 64),
    ("gqa5_hd128", 10, 2, 128, 261, 96),
    ("gqa8_hd64", 16, 2, 64, 130, 130),
    ("gqa1_long_split", 2, 2, 128, 2100, 37),
]


@pytest.mark.parametrize("name,nh,nkv,hd,T,chunk", CASES)
def test_bf16_prefill_matches_oracle(name, nh, nkv, hd, T, chunk):
    say(f"bf16 prefill {name}: nh={nh} nkv={nkv} hd={hd} T={T} chunk={chunk}")
    w = wl.Workload(name=name, dtype=wl.BF16, n_heads=nh, n_kv=nkv, head_dim=hd, seed=21,
                    prompt_len=T, chunk=chunk)
    d = wl.gen_prefill(w)
    run = runner.ChunkedPrefill(w, d, device=DEV)
    run.run_all()
    torch.cuda.synchronize()
    ref = oracle_prefill_packed(w, d, chunk)
    check_bf16_rows(np64(run.gather("out")), ref["out"], name)
    # the rotated queries and the cache equal the oracle's rounded values
    assert np.array_equal(_bits(run.gather("q_rot")), _to_dtype_bits(ref["q_rot"], torch.bfloat16))
    kc_ref, vc_ref = ref["caches"][0]
    assert np.array_equal(_bits(run.k_cache[0]), _to_dtype_bits(kc_ref, torch.bfloat16))
    assert np.array_equal(_bits(run.v_cache[0]), _to_dtype_bits(vc_ref, torch.bfloat16))


def test_bf16_varlen_qknorm_partial_rotary():
    w = wl.Workload(name="varlen", dtype=wl.BF16, n_heads=10, n_kv=2, head_dim=128, seed=23,
                    base=1e6, rotary_dim=64, norm_style=wl.NORM_W, n_seq=4, len_range=(40, 700),
                    chunk=256, cap=700)
    say(f"bf16 varlen {w}")
    d = wl.gen_prefill(w)
    run = runner.ChunkedPrefill(w, d, device=DEV)
    run.run_all()
    torch.cuda.synchronize()
    ref = oracle_prefill_packed(w, d, 256)
    check_bf16_rows(np64(run.gather("out")), ref["out"], "varlen")


def test_bf16_varlen_many_sequences_wide_tiles():
    # 32 prompts x 8 KV groups give enough 256-row tiles for the 8-wave,
    # deeper-prefetch variant; ragged lengths cover empty and partial tiles
    w = wl.Workload(name="wide", dtype=wl.BF16, n_heads=32, n_kv=8, head_dim=128, seed=26,
                    n_seq=32, len_range=(1, 200), chunk=64, cap=200)
    say(f"bf16 varlen 32 sequences {w}")
    d = wl.gen_prefill(w)
    run = runner.ChunkedPrefill(w, d, device=DEV)
    assert any(api.prefill_workspace_bytes(s["batch"], 32, 8, 128) == 0 for s in run.steps)
    run.run_all()
    torch.cuda.synchronize()
    ref = oracle_prefill_packed(w, d, 64)
    check_bf16_rows(np64(run.gather("out")), ref["out"], "wide")


def test_bf16_chunked_equals_sequential():
    w = wl.Workload(name="seq", dtype=wl.BF16, n_heads=8, n_kv=2, head_dim=128, seed=24,
                    prompt_len=160, chunk=64)
    d = wl.gen_prefill(w)
    outs = {}
    for chunk in (1, 2, 64, 160):
        run = runner.ChunkedPrefill(w, d, device=DEV, chunk=chunk)
        run.run_all()
        torch.cuda.synchronize()
        outs[chunk] = np64(run.gather("out"))
        caches = (_bits(run.k_cache), _bits(run.v_cache))
        if chunk == 1:
            ref_caches = caches
        else:
            # the cache does not depend on the chunking, bit for bit
            assert np.array_equal(caches[0], ref_caches[0])
            assert np.array_equal(caches[1], ref_caches[1])
    ref = oracle_prefill_packed(w, d, 1)["out"]
    for chunk, o in outs.items():
        check_bf16_rows(o, ref, f"chunk {chunk}")


def test_empty_and_single_token():
    w = wl.Workload(name="one", dtype=wl.BF16, n_heads=4, n_kv=1, head_dim=64, seed=25,
                    prompt_len=1, chunk=1)
    d = wl.gen_prefill(w)
    run = runner.ChunkedPrefill(w, d, device=DEV)
    run.run_all()
    torch.cuda.synchronize()
    # position 0 attends only itself: the output is V0 exactly
    v0 = np64(d["v"][0])
    got = np64(run.gather("out"))[0]
    for h in range(4):
        assert np.array_equal(got[h], v0[0])
    # an empty batch is a no-op
    out = torch.full((1, 4, 64), 7.0, device=DEV)
    empty = api.Batch([0], [0], device=DEV)
    api.prefill_chunk(run.steps[0]["q_rot"], run.k_cache, run.v_cache, empty, w.scale, out)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)


# ------------------------------------------------------------------ bf16 decode

@pytest.mark.parametrize("nh,nkv,hd,ld_mult", [(16, 4, 128, 32), (16, 2, 64, 1), (8, 8, 128, 1),
                                                (40, 8, 128, 32), (32, 8, 128, 1)])
def test_bf16_decode_matches_oracle(nh, nkv, hd, ld_mult):
    ctx = [1, 63, 64, 65, 1025, 3000]
    w = wl.Workload(name="dec", dtype=wl.BF16, n_heads=nh, n_kv=nkv, head_dim=hd, seed=31,
                    n_seq=len(ctx), decode=True, ctx_range=(1, 3000), cap=3072, want_probs=True)
    say(f"bf16 decode nh={nh} nkv={nkv} hd={hd} ctx={ctx}")
    d = wl.gen_decode(w)
    d["ctx"] = ctx
    step = runner.DecodeStep(w, d, device=DEV, probs_ld_multiple=ld_mult)
    step.probs.fill_(float("nan"))
    step.run()
    torch.cuda.synchronize()
    f = oracle_table(w)
    got_o = np64(step.out)
    got_p = np64(step.probs)
    for b, c in enumerate(ctx):
        pos = np.array([c - 1])
        kc = np64(d["k_cache"][b])[:, :c].copy()
        vc = np64(d["v_cache"][b])[:, :c].copy()
        kc[:, c - 1] = oracle.finish_heads(np64(d["k"][b:b + 1]), pos, f, w.rd,
                                           store=oracle.STORE_BF16)[0]
        vc[:, c - 1] = np64(d["v"][b])
        q = oracle.finish_heads(np64(d["q"][b:b + 1]), pos, f, w.rd, store=oracle.STORE_BF16)
        o, P = oracle.attend(q, kc, vc, pos, w.scale, want_probs=True)
        check_bf16_rows(got_o[b], o[0], f"seq {b} ctx {c}")
        pg = got_p[b, :, :c]
        assert np.all(np.isnan(got_p[b, :, c:])), "entries past ctx must stay untouched"
        check_probs(pg, P[0], True, f"seq {b} ctx {c}")
    # the new token's K/V rows were appended at ctx-1
    for b, c in enumerate(ctx):
        assert np.array_equal(_bits(step.v_cache[b, :, c - 1]), _bits(d["v"][b]))


@pytest.mark.parametrize("nh,nkv,parts_per_row,spike", [(32, 2, 1, False), (16, 2, 2, False),
                                                         (32, 2, 1, True), (16, 4, 1, True)])
def test_bf16_decode_small_workspace(nh, nkv, parts_per_row, spike):
    """A workspace for fewer parts makes each part longer than the on-chip
    raw-score buffer of a wide group (16, 8 or 4 heads), so the split kernel
    writes values out several times per part.  With a spike, a late key's
    score for one head of each group exceeds everything before it by far, so
    the running maximum moves after values were written and those are
    rescaled."""
    ctx = [3000, 700, 1, 2049]
    hd = 128
    w = wl.Workload(name="dec-ws", dtype=wl.BF16, n_heads=nh, n_kv=nkv, head_dim=hd, seed=37,
                    n_seq=len(ctx), decode=True, ctx_range=(1, 3000), cap=3072, want_probs=True)
    say(f"bf16 decode small workspace nh={nh} nkv={nkv} parts/row={parts_per_row} spike={spike} ctx={ctx}")
    d = wl.gen_decode(w)
    d["ctx"] = ctx
    if spike:
        # key c-100 of sequence b, for KV group g, is 1.5x the rotated query
        # of head g*G (a score near 16 in log2 units above the rest)
        f = oracle_table(w)
        G = nh // nkv
        for b, c in enumerate(ctx):
            if c < 1000:
                continue
            q = oracle.finish_heads(np64(d["q"][b:b + 1]), np.array([c - 1]), f, w.rd,
                                    store=oracle.STORE_BF16)[0]
            for g in range(nkv):
                d["k_cache"][b, g, c - 100] = torch.from_numpy(1.5 * q[g * G]).to(torch.bfloat16)
    step = runner.DecodeStep(w, d, device=DEV, probs_ld_multiple=1)
    step.workspace = torch.empty(len(ctx) * nh * (hd + 4) * parts_per_row, dtype=torch.float32,
                                 device=DEV)
    step.probs.fill_(float("nan"))
    step.run()
    torch.cuda.synchronize()
    f = oracle_table(w)
    got_o = np64(step.out)
    got_p = np64(step.probs)
    for b, c in enumerate(ctx):
        pos = np.array([c - 1])
        kc = np64(d["k_cache"][b])[:, :c].copy()
        vc = np64(d["v_cache"][b])[:, :c].copy()
        kc[:, c - 1] = oracle.finish_heads(np64(d["k"][b:b + 1]), pos, f, w.rd,
                                           store=oracle.STORE_BF16)[0]
        vc[:, c - 1] = np64(d["v"][b])
        q = oracle.finish_heads(np64(d["q"][b:b + 1]), pos, f, w.rd, store=oracle.STORE_BF16)
        o, P = oracle.attend(q, kc, vc, pos, w.scale, want_probs=True)
        check_bf16_rows(got_o[b], o[0], f"seq {b} ctx {c}")
        assert np.all(np.isnan(got_p[b, :, c:])), "entries past ctx must stay untouched"
        pg = got_p[b, :, :c]
        check_probs(pg, P[0], True, f"seq {b} ctx {c}")


# ------------------------------------------------------------------ sliding window

WINDOW_CASES = [
    # name, nh, nkv, hd, T, chunk, window
    ("w100_chunk128", 8, 2, 128, 700, 128, 100),      # window below the chunk
    ("w300_chunk256", 8, 2, 128, 700, 256, 300),
    ("w64_mha_hd64", 3, 3, 64, 500, 64, 64),          # window = one key tile
    ("w1_gqa8_hd64", 16, 2, 64, 400, 130, 1),         # every row reads only itself
    ("w777_long_split", 2, 2, 128, 2100, 37, 777),    # small chunks, split key range
    ("w2000_long_split", 8, 8, 128, 2100, 64, 2000),
]


@pytest.mark.parametrize("name,nh,nkv,hd,T,chunk,window", WINDOW_CASES)
def test_bf16_prefill_window_matches_oracle(name, nh, nkv, hd, T, chunk, window):
    say(f"bf16 prefill window {name}: nh={nh} nkv={nkv} hd={hd} T={T} chunk={chunk} W={window}")
    w = wl.Workload(name=name, dtype=wl.BF16, n_heads=nh, n_kv=nkv, head_dim=hd, seed=41,
                    prompt_len=T, chunk=chunk, window=window)
    d = wl.gen_prefill(w)
    run = runner.ChunkedPrefill(w, d, device=DEV)
    run.run_all()
    torch.cuda.synchronize()
    got = np64(run.gather("out"))
    ref = oracle_prefill_packed(w, d, chunk)
    check_bf16_rows(got, ref["out"], name)
    if window == 1:
        # one key: the output is that position's V row exactly
        v = np64(d["v"])
        for h in range(nh):
            assert np.array_equal(got[:, h], v[:, h // (nh // nkv)])


def test_bf16_prefill_window_varlen_and_wide_window():
    """Ragged prompts with a window, in 128- and 256-row workgroups; a window
    at least as long as every prompt gives the unwindowed result bit for bit."""
    for n_seq, chunk, window in ((4, 256, 200), (32, 64, 50)):
        w = wl.Workload(name="varlen-w", dtype=wl.BF16, n_heads=32 if n_seq == 32 else 10,
                        n_kv=8 if n_seq == 32 else 2, head_dim=128, seed=43, base=1e6,
                        rotary_dim=64, norm_style=wl.NORM_W, n_seq=n_seq,
                        len_range=(1, 700), chunk=chunk, cap=700, window=window)
        say(f"bf16 varlen window {w}")
        d = wl.gen_prefill(w)
        run = runner.ChunkedPrefill(w, d, device=DEV)
        run.run_all()
        torch.cuda.synchronize()
        ref = oracle_prefill_packed(w, d, chunk)
        check_bf16_rows(np64(run.gather("out")), ref["out"], f"varlen window {window}")
    w = wl.Workload(name="wide-w", dtype=wl.BF16, n_heads=8, n_kv=2, head_dim=128, seed=44,
                    prompt_len=600, chunk=96)
    d = wl.gen_prefill(w)
    outs = []
    for window in (0, 600, 10 ** 6):
        run = runner.ChunkedPrefill(w.replace(window=window), d, device=DEV)
        run.run_all()
        torch.cuda.synchronize()
        outs.append(_bits(run.gather("out")))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def test_f32_prefill_window_and_probs():
    w = wl.CONFIGS["c0_f32_small"].replace(window=20)
    d = wl.gen_prefill(w)
    ref = oracle_prefill_packed(w, d, 16, want_probs=True)
    for chunk in (16, 1, 64):
        run = runner.ChunkedPrefill(w, d, device=DEV, chunk=chunk)
        run.run_all()
        torch.cuda.synchronize()
        check_f32(np64(run.gather("out")), ref["out"], f"f32 window chunk {chunk}")


def _decode_reference(w, d, b, c):
    return oracle_decode_row(w, d, b, c)


@pytest.mark.parametrize("dtype,nh,nkv,window,parts_per_row", [
    (wl.BF16, 32, 8, 1, 0), (wl.BF16, 32, 8, 33, 0), (wl.BF16, 16, 2, 100, 0),
    (wl.BF16, 40, 8, 1024, 0), (wl.BF16, 8, 8, 5000, 0),
    (wl.BF16, 32, 2, 2500, 1),             # one part per row, longer than the on-chip buffer
    (wl.F32, 8, 2, 100, 0)])
def test_decode_window_matches_oracle(dtype, nh, nkv, window, parts_per_row):
    ctx = [1, 63, 64, 65, 1025, 3000, 2049, 97]
    hd = 128
    w = wl.Workload(name="dec-w", dtype=dtype, n_heads=nh, n_kv=nkv, head_dim=hd, seed=47,
                    n_seq=len(ctx), decode=True, ctx_range=(1, 3000), cap=3072, want_probs=True,
                    window=window)
    say(f"decode window {dtype} nh={nh} nkv={nkv} W={window} parts/row={parts_per_row} ctx={ctx}")
    d = wl.gen_decode(w)
    d["ctx"] = ctx
    step = runner.DecodeStep(w, d, device=DEV, probs_ld_multiple=1)
    if parts_per_row:
        step.workspace = torch.empty(len(ctx) * nh * (hd + 4) * parts_per_row,
                                     dtype=torch.float32, device=DEV)
    step.probs.fill_(float("nan"))
    step.run()
    torch.cuda.synchronize()
    got_o = np64(step.out)
    got_p = np64(step.probs)
    for b, c in enumerate(ctx):
        o, P = _decode_reference(w, d, b, c)
        if dtype == wl.BF16:
            check_bf16_rows(got_o[b], o, f"seq {b} ctx {c}")
        else:
            check_f32(got_o[b], o, f"seq {b} ctx {c}")
        assert np.all(np.isnan(got_p[b, :, c:])), "entries past ctx must stay untouched"
        pg = got_p[b, :, :c]
        first = max(0, c - window)
        assert np.all(pg[:, :first] == 0.0), "keys before the window get probability 0"
        if window == 1:
            assert np.all(pg[:, c - 1] == 1.0)
        check_probs(pg, P, dtype == wl.BF16, f"seq {b} ctx {c}")


# ------------------------------------------------------------------ ring cache

RING_CASES = [
    # name, nh, nkv, hd, T, chunk, window, ring rows (>= window + chunk - 1, a multiple of 64)
    ("ring256_w100_c128", 8, 2, 128, 700, 128, 100, 256),
    ("ring832_w777_split", 2, 2, 128, 2100, 37, 777, 832),
    ("ring256_w64_hd64", 16, 2, 64, 400, 130, 64, 256),
    ("ring192_exact", 8, 8, 128, 500, 64, 129, 192),          # window + chunk - 1 = ring
]


@pytest.mark.parametrize("name,nh,nkv,hd,T,chunk,window,ring", RING_CASES)
def test_bf16_prefill_ring_matches_oracle(name, nh, nkv, hd, T, chunk, window, ring):
    """Prefill over a ring cache of `ring` rows: every output equals the
    windowed run over a full-length cache bit for bit, and the oracle's ring
    prefill; every ring row holds the oracle's rounded K (V bit copies) of the
    latest position congruent to it."""
    say(f"bf16 prefill ring {name}: nh={nh} nkv={nkv} hd={hd} T={T} chunk={chunk} W={window} R={ring}")
    w = wl.Workload(name=name, dtype=wl.BF16, n_heads=nh, n_kv=nkv, head_dim=hd, seed=61,
                    prompt_len=T, chunk=chunk, window=window)
    d = wl.gen_prefill(w)
    lin = runner.ChunkedPrefill(w, d, device=DEV)
    lin.run_all()
    wr = w.replace(ring=True, cap=ring)
    dr = dict(d, cap=ring)
    run = runner.ChunkedPrefill(wr, dr, device=DEV)
    assert run.k_cache.shape[2] == ring
    run.run_all()
    torch.cuda.synchronize()
    assert np.array_equal(_bits(run.gather("out")), _bits(lin.gather("out")))
    ref = oracle_prefill_packed(wr, dr, chunk)
    check_bf16_rows(np64(run.gather("out")), ref["out"], name)
    kc_ref, vc_ref = ref["caches"][0]
    assert not np.isnan(kc_ref).any()
    assert np.array_equal(_bits(run.k_cache[0]), _to_dtype_bits(kc_ref, torch.bfloat16))
    assert np.array_equal(_bits(run.v_cache[0]), _to_dtype_bits(vc_ref, torch.bfloat16))


def test_f32_prefill_ring():
    # f32 takes any ring length (no tile alignment)
    w = wl.CONFIGS["c0_f32_small"].replace(window=20, ring=True, cap=40)
    d = wl.gen_prefill(w)
    d = dict(d, cap=40)
    ref = oracle_prefill_packed(w, d, 16)
    run = runner.ChunkedPrefill(w, d, device=DEV, chunk=16)
    run.run_all()
    torch.cuda.synchronize()
    check_f32(np64(run.gather("out")), ref["out"], "f32 ring")
    assert np.array_equal(np64(run.k_cache[0]), ref["caches"][0][0])


def test_ring_capacity_errors():
    w = wl.Workload(name="ring-err", dtype=wl.BF16, n_heads=4, n_kv=2, head_dim=64, seed=62,
                    prompt_len=300, chunk=100, window=100, ring=True, cap=192)
    d = wl.gen_prefill(w)
    run = runner.ChunkedPrefill(w, dict(d, cap=192), device=DEV)
    run.run_step(0)          # positions 0..99: the ring has not wrapped
    # positions 100..199 wrap the 192-row ring, and writing a chunk before it
    # attends needs 100 + 100 - 1 = 199 rows
    with pytest.raises(RuntimeError, match="capacity"):
        run.run_step(1)
    torch.cuda.synchronize()


@pytest.mark.parametrize("dtype,nh,nkv,window,ring,parts_per_row", [
    (wl.BF16, 32, 8, 100, 128, 0), (wl.BF16, 16, 2, 128, 128, 0), (wl.BF16, 40, 8, 1000, 1024, 0),
    (wl.BF16, 32, 2, 2500, 2600, 1),      # one long part per row
    (wl.F32, 8, 2, 100, 100, 0)])
def test_decode_ring_matches_oracle(dtype, nh, nkv, window, ring, parts_per_row):
    """Decode over a ring of `ring` rows: position j in row j mod ring (the
    drawn cache rows stand for the latest positions congruent to them)."""
    ctx = [1, 63, 64, 65, 1025, 3000, 2049, 97]
    hd = 128
    w = wl.Workload(name="dec-ring", dtype=dtype, n_heads=nh, n_kv=nkv, head_dim=hd, seed=63,
                    n_seq=len(ctx), decode=True, ctx_range=(1, 3000), cap=ring, want_probs=True,
                    window=window, ring=True)
    say(f"decode ring {dtype} nh={nh} nkv={nkv} W={window} R={ring} parts/row={parts_per_row}")
    d = wl.gen_decode(w)
    d["ctx"] = ctx
    step = runner.DecodeStep(w, d, device=DEV, probs_ld_multiple=1)
    if parts_per_row:
        step.workspace = torch.empty(len(ctx) * nh * (hd + 4) * parts_per_row,
                                     dtype=torch.float32, device=DEV)
    step.probs.fill_(float("nan"))
    step.run()
    torch.cuda.synchronize()
    got_o = np64(step.out)
    got_p = np64(step.probs)
    for b, c in enumerate(ctx):
        o, P = oracle_decode_row(w, d, b, c)
        if dtype == wl.BF16:
            check_bf16_rows(got_o[b], o, f"seq {b} ctx {c}")
        else:
            check_f32(got_o[b], o, f"seq {b} ctx {c}")
        assert np.all(np.isnan(got_p[b, :, c:]))
        pg = got_p[b, :, :c]
        assert np.all(pg[:, :max(0, c - window)] == 0.0)
        check_probs(pg, P, dtype == wl.BF16, f"seq {b} ctx {c}")
        # the new token's row went to row (c-1) mod ring
        assert np.array_equal(_bits(step.v_cache[b, :, (c - 1) % ring]), _bits(d["v"][b]))


# ------------------------------------------------------------------ gates and V-norm

GATE_CASES = [
    # name, nh, nkv, hd, T, chunk, gate mode, v_norm
    ("sigmoid_vnorm", 8, 2, 128, 300, 128, 1, True),
    ("softplus_head", 10, 2, 128, 261, 96, 2, False),
    ("softplus_elem_hd64", 16, 2, 64, 130, 130, 3, True),
    ("sigmoid_long_split", 2, 2, 128, 2100, 37, 1, False),     # gate in the combine kernel
]


@pytest.mark.parametrize("name,nh,nkv,hd,T,chunk,mode,v_norm", GATE_CASES)
def test_bf16_prefill_gates_and_vnorm(name, nh, nkv, hd, T, chunk, mode, v_norm):
    say(f"bf16 prefill gate {name}: mode={mode} v_norm={v_norm}")
    w = wl.Workload(name=name, dtype=wl.BF16, n_heads=nh, n_kv=nkv, head_dim=hd, seed=81,
                    prompt_len=T, chunk=chunk, gate_mode=mode, v_norm=v_norm)
    d = wl.gen_prefill(w)
    run = runner.ChunkedPrefill(w, d, device=DEV)
    run.run_all()
    torch.cuda.synchronize()
    ref = oracle_prefill_packed(w, d, chunk)
    check_bf16_rows(np64(run.gather("out")), ref["out"], name, gain=gain_of(w, d["gate"], ref["out"].shape))
    kc_ref, vc_ref = ref["caches"][0]
    want_v = _to_dtype_bits(vc_ref, torch.bfloat16)
    mism = int((_bits(run.v_cache[0]) != want_v).sum())
    assert mism <= max(1, want_v.size // 1_000_000), f"V cache: {mism} rows differ"
    if not v_norm:
        assert mism == 0


def test_gate_view_of_raw_query_projection():
    """The Qwen3.5 layout: each head's raw projection rows [q(hd); gate(hd)];
    a gate read in place through gate_ld = 2*hd gives the same bits as the
    gate copied out."""
    w = wl.Workload(name="qwen-gate", dtype=wl.BF16, n_heads=8, n_kv=2, head_dim=128, seed=82,
                    prompt_len=200, chunk=200, gate_mode=1)
    d = wl.gen_prefill(w)
    run = runner.ChunkedPrefill(w, d, device=DEV)
    run.run_all()
    s = run.steps[0]
    raw = torch.cat([s["q"], s["gate"]], dim=-1)          # [T][nh][2*hd]
    out2 = torch.empty_like(s["out"])
    api.prefill_chunk(s["q_rot"], run.k_cache, run.v_cache, s["batch"], w.scale, out2,
                      run.workspace, gate=raw[..., 128:], gate_mode=api.GATE_SIGMOID)
    torch.cuda.synchronize()
    assert torch.equal(out2, s["out"])


def test_f32_prefill_and_decode_gates():
    for mode in (1, 2, 3):
        w = wl.CONFIGS["c0_f32_small"].replace(gate_mode=mode, v_norm=mode == 3)
        d = wl.gen_prefill(w)
        ref = oracle_prefill_packed(w, d, 16)
        run = runner.ChunkedPrefill(w, d, device=DEV)
        run.run_all()
        torch.cuda.synchronize()
        check_f32(np64(run.gather("out")), ref["out"], f"f32 prefill gate {mode}")


@pytest.mark.parametrize("dtype,mode,v_norm,window", [
    (wl.BF16, 1, True, 0), (wl.BF16, 2, False, 100), (wl.BF16, 3, False, 0), (wl.F32, 1, True, 0),
    (wl.F32, 2, False, 0)])
def test_decode_gates_and_vnorm(dtype, mode, v_norm, window):
    ctx = [1, 63, 64, 65, 1025, 3000]
    w = wl.Workload(name="dec-gate", dtype=dtype, n_heads=32, n_kv=8, head_dim=128, seed=83,
                    n_seq=len(ctx), decode=True, ctx_range=(1, 3000), cap=3072, want_probs=True,
                    gate_mode=mode, v_norm=v_norm, window=window)
    say(f"decode gate {dtype} mode={mode} v_norm={v_norm} W={window}")
    d = wl.gen_decode(w)
    d["ctx"] = ctx
    step = runner.DecodeStep(w, d, device=DEV, probs_ld_multiple=1)
    step.run()
    torch.cuda.synchronize()
    got_o = np64(step.out)
    got_p = np64(step.probs)
    for b, c in enumerate(ctx):
        o, P = oracle_decode_row(w, d, b, c)
        if dtype == wl.BF16:
            gain = gain_of(w, d["gate"][b] if w.gate_mode else None, o.shape)
            check_bf16_rows(got_o[b], o, f"seq {b} ctx {c}", gain=gain)
        else:
            check_f32(got_o[b], o, f"seq {b} ctx {c}")
        # the probabilities are not gated
        check_probs(got_p[b, :, :c], P, dtype == wl.BF16, f"seq {b} ctx {c}")


# ------------------------------------------------------------------ chunks of 1-2 tokens

@pytest.mark.parametrize("nh,nkv,n_new,window,ring,gate", [
    (32, 8, 2, 0, 0, 0), (32, 8, 1, 0, 0, 0), (16, 2, 2, 0, 0, 1), (40, 8, 2, 100, 0, 0),
    (8, 8, 2, 0, 0, 2), (32, 8, 2, 1000, 1088, 0), (64, 8, 2, 0, 0, 0), (32, 2, 2, 0, 0, 0)])
def test_small_chunk_path_matches_oracle(nh, nkv, n_new, window, ring, gate):
    """Chunks of at most two tokens run on the decode kernels (query rows =
    heads x tokens, up to 16: 64/8 heads x 2 tokens is the widest); wider
    groups (32/2 x 2) take the prefill kernel.  Against the oracle, and against the prefill
    kernel run on the same batch (a workspace too small for the decode
    kernels' parts)."""
    ctx = [2, 3, 63, 64, 65, 1025, 3000, 2049, 97] if n_new == 2 else [1, 2, 64, 1025, 3000]
    hd = 128
    cap = ring or 3072
    w = wl.Workload(name="small-chunk", dtype=wl.BF16, n_heads=nh, n_kv=nkv, head_dim=hd, seed=91,
                    n_seq=len(ctx), decode=True, ctx_range=(2, 3000), cap=cap, new_tokens=n_new,
                    window=window, ring=bool(ring), gate_mode=gate)
    say(f"small chunk nh={nh} nkv={nkv} n={n_new} W={window} ring={ring} gate={gate}")
    d = wl.gen_decode(w)
    d["ctx"] = ctx
    step = runner.VerifyStep(w, d, device=DEV)
    step.run()
    torch.cuda.synchronize()
    got = np64(step.out).reshape(len(ctx), n_new, nh, hd)
    for b, c in enumerate(ctx):
        ref = oracle_verify_rows(w, d, b, c)
        g = d["gate"][b * n_new:(b + 1) * n_new] if gate else None
        check_bf16_rows(got[b], ref, f"seq {b} ctx {c}", gain=gain_of(w, g, ref.shape))
    if not ring:
        # the prefill kernel on the same batch (the cache already holds the rows)
        small = torch.empty(4, dtype=torch.float32, device=DEV)
        ref = step.out.clone()
        step.attend(workspace=small)
        torch.cuda.synchronize()
        check_bf16_rows(np64(step.out), np64(ref), "decode kernels vs prefill kernel")


# ------------------------------------------------------------------ importance

@pytest.mark.parametrize("dtype,nh,nkv", [(wl.BF16, 32, 8), (wl.F32, 32, 8), (wl.BF16, 40, 8),
                                          (wl.BF16, 10, 2), (wl.F32, 40, 8)])
def test_decode_importance_matches_oracle(dtype, nh, nkv):
    """Per-position importance after a decode step: the sum over heads of
    the probabilities.  Against the GPU's own probabilities summed in head
    order in float (bit for bit), against the oracle's importance (within the
    probabilities' tolerance, summed over heads), accumulating twice doubles
    it exactly, and entries past ctx stay untouched.  40 and 10 heads are not
    multiples of the kernel's 16-head load groups, so its leftover-heads loop
    runs too."""
    ctx = [1, 63, 64, 65, 1025, 3000]
    hd = 128
    w = wl.Workload(name="imp", dtype=dtype, n_heads=nh, n_kv=nkv, head_dim=hd, seed=43,
                    n_seq=len(ctx), decode=True, ctx_range=(1, 3000), cap=3072, want_probs=True)
    say(f"decode importance dtype={dtype} heads {nh}/{nkv} ctx={ctx}")
    d = wl.gen_decode(w)
    d["ctx"] = ctx
    step = runner.DecodeStep(w, d, device=DEV, probs_ld_multiple=1)
    step.run()
    imp = torch.full((len(ctx), 3100), float("nan"), device=DEV)
    api.decode_importance(step.probs, step.ctx, step.max_ctx, imp, accumulate=False)
    torch.cuda.synchronize()
    gp = step.probs.detach().cpu().numpy()
    gi = imp.detach().cpu().numpy()
    f = oracle_table(w)
    for b, c in enumerate(ctx):
        own = np.zeros(c, dtype=np.float32)
        for h in range(nh):
            own += gp[b, h, :c]
        assert np.array_equal(gi[b, :c], own), f"seq {b}: not the head-ordered float sum"
        assert np.all(np.isnan(gi[b, c:])), "entries past ctx must stay untouched"
        pos = np.array([c - 1])
        kc = np64(d["k_cache"][b])[:, :c].copy()
        vc = np64(d["v_cache"][b])[:, :c].copy()
        store = store_of(w)
        kc[:, c - 1] = oracle.finish_heads(np64(d["k"][b:b + 1]), pos, f, w.rd, store=store)[0]
        vc[:, c - 1] = np64(d["v"][b])
        q = oracle.finish_heads(np64(d["q"][b:b + 1]), pos, f, w.rd, store=store)
        _, P = oracle.attend(q, kc, vc, pos, w.scale, want_probs=True)
        ref = oracle.head_importance(P[0], c)
        # the heads' probability bounds added up, plus the float sum's rounding
        if dtype == wl.BF16:
            tol = (PROB_REL_TOL + 2e-6) * ref + PROB_ABS_FRAC * P[0].max(-1).sum()
        else:
            tol = np.full(c, nh * 1e-4)
        err = np.abs(gi[b, :c] - ref)
        say(f"  seq {b} ctx {c}: worst |d imp|/tol {float(np.max(err / tol)):.3f}, sum {gi[b, :c].sum():.6f}")
        assert np.all(err <= tol)
        assert abs(float(gi[b, :c].astype(np.float64).sum()) - nh) <= 1e-4 * nh
    # accumulating adds the same vector again: exactly twice the first
    first = imp.clone()
    api.decode_importance(step.probs, step.ctx, step.max_ctx, imp, accumulate=True)
    torch.cuda.synchronize()
    for b, c in enumerate(ctx):
        assert torch.equal(imp[b, :c], 2 * first[b, :c])


# ------------------------------------------------------------------ graphs

def test_graph_replay_matches_eager():
    w = wl.Workload(name="graph", dtype=wl.BF16, n_heads=8, n_kv=2, head_dim=128, seed=41,
                    prompt_len=512, chunk=128)
    d = wl.gen_prefill(w)
    run = runner.ChunkedPrefill(w, d, device=DEV)
    run.run_all()
    torch.cuda.synchronize()
    eager = run.gather("out").clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        run.run_all()  # warm-up on the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            run.run_all()
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(4):
        for st in run.steps:
            st["out"].fill_(float("nan"))
        junk = torch.randn(1 << 20, device=DEV).sum()  # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        assert torch.equal(run.gather("out"), eager), f"replay {rep} differs from eager"
