"""GPU parity of the chunked prefill (gdn_prefill_chunked) with the fp64
oracle, through the C ABI, on both paths (the fused single-pass kernel, run
without a workspace, and the two-pass prep + state kernels, run with one):
small cases spanning several chunks and ragged tails in every kernel variant,
edge lengths, unaligned starts, checkpoints and bitwise resume, segmented
workspaces, continuation into decode, and the full-size workloads.
"""
import os

import numpy as np
import pytest
import torch

from linear_attention_recurrence_causal_amd import inputs as I
from tests.helpers import (finite, oracle_decode, oracle_prefill, rel, to_dev, tols,
                           TOL_BF16_OUT, TOL_BF16_STATE)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def G():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from linear_attention_recurrence_causal_amd import gdn
    return gdn


PATHS = ["fused", "split"]
WAVE_VARS = ("GDN_PREFILL_WAVES", "GDN_PREFILL_STATE_WAVES")


@pytest.fixture
def waves():
    """Force a kernel variant (2, 4 or 8 waves = 32, 64 or 128 state columns
    per workgroup of the fused or the state kernel) for one test, then
    restore the size-based choice."""
    old = {k: os.environ.get(k) for k in WAVE_VARS}

    def set_(n):
        for k in WAVE_VARS:
            if n is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = str(n)
    yield set_
    for k, v in old.items():
        if v is None:
            os.environ.pop(k, None)
        else:
            os.environ[k] = v


def cfg_of(G, w, precision=0):
    return G.Config(batch=w.batch, num_k_heads=w.num_k_heads, num_v_heads=w.num_v_heads, precision=precision)


def gpu_prefill(G, w, d, seq=slice(None), start_pos=0, conv_in="init", rec_in="init",
                ckpt_interval=0, ckpt_buf=None, rec_out=None, path="split", workspace="auto", precision=0):
    """path "fused": no workspace; "split": the given workspace ("auto" = the
    whole call in one segment); precision: gdn_precision."""
    c = cfg_of(G, w, precision)
    ws = None if path == "fused" else workspace
    # a workspace selects the two-pass path; "split" keeps it selected even
    # if the environment asks for the fused kernel
    old_env = os.environ.get("GDN_PREFILL_PATH")
    os.environ["GDN_PREFILL_PATH"] = "split" if path == "split" else "auto"
    cin = d["conv_state"] if conv_in == "init" else conv_in
    rin = d["rec_state"] if rec_in == "init" else rec_in
    out, conv, S = G.prefill_chunked(c, d["qkv"][:, seq].contiguous(), d["a"][:, seq].contiguous(),
                                     d["b"][:, seq].contiguous(), d["conv_w"], d["A_log"],
                                     d["dt_bias"], cin, rin, start_pos=start_pos,
                                     ckpt_interval=ckpt_interval, ckpt_buf=ckpt_buf,
                                     rec_state_out=rec_out, workspace=ws)
    if old_env is None:
        os.environ.pop("GDN_PREFILL_PATH", None)
    else:
        os.environ["GDN_PREFILL_PATH"] = old_env
    torch.cuda.synchronize()
    return out, conv, S


def local_rel(x, ref, window=64):
    """Worst relative L2 over every `window`-token run of every (sequence,
    head): x, ref [B, L, H, d].  A fault confined to a few chunks or heads
    cannot hide in the global norm.  A run whose reference is zero is held
    to the absolute size of x there; below 1e-30 (fp32 range) the
    difference counts as absolute."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    B, L, H, d = ref.shape
    n = (L + window - 1) // window
    pad = n * window - L
    if pad:
        z = np.zeros((B, pad, H, d))
        x, ref = np.concatenate([x, z], 1), np.concatenate([ref, z], 1)
    num = ((x - ref) ** 2).reshape(B, n, window, H, d).sum(axis=(2, 4))
    den = (ref ** 2).reshape(B, n, window, H, d).sum(axis=(2, 4))
    return float(np.sqrt(num / np.maximum(den, 1e-60)).max())


def state_rel_per_head(s, ref):
    """Worst relative L2 of the state over the (sequence, head) pairs: s, ref
    [B, H, d_k, d_v].  A state that has decayed below the fp32 range (norm
    under 1e-30) is held to that absolute size instead."""
    s = np.asarray(s, np.float64)
    ref = np.asarray(ref, np.float64)
    num = ((s - ref) ** 2).sum(axis=(2, 3))
    den = (ref ** 2).sum(axis=(2, 3))
    return float(np.sqrt(num / np.maximum(den, 1e-60)).max())


def compare(tag, w, out, conv, S, ref, heads=None, batch_idx=None):
    """The bars on the whole compared tensors, on every 64-token run of every
    compared (sequence, head), and on every head's state."""
    bi = list(range(w.batch)) if batch_idx is None else list(batch_idx)
    hs = list(range(w.num_v_heads)) if heads is None else list(heads)
    o = out[bi][:, :, hs].double().cpu().numpy()
    s = S[bi][:, hs].double().cpu().numpy()
    t_out, t_state = tols(w)
    e_out, e_state = rel(o, ref["out"]), rel(s, ref["S"])
    l_out, l_state = local_rel(o, ref["out"]), state_rel_per_head(s, ref["S"])
    print(f"[{tag}] out rel {e_out:.3e}, worst 64-token run {l_out:.3e} (bar {t_out}); "
          f"state rel {e_state:.3e}, worst head {l_state:.3e} (bar {t_state})", flush=True)
    assert e_out <= t_out and e_state <= t_state
    assert l_out <= t_out and l_state <= t_state
    assert np.array_equal(I.to_numpy_io(conv[bi]), ref["conv_tail"])
    assert finite(out, S)


def small(**kw):
    base = dict(name="small", batch=2, seq_len=200, num_k_heads=2, num_v_heads=4, seed=21)
    base.update(kw)
    return I.Workload(**base)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("nw", [2, 4, 8])
@pytest.mark.parametrize("init", [False, True])
def test_prefill_small_all_variants(G, waves, path, nw, init):
    """200 tokens = 3 full chunks + a ragged 8-token tail, two sequences."""
    waves(nw)
    w = small(init_state=init, seed=21 + init)
    inp = I.generate(w)
    out, conv, S = gpu_prefill(G, w, to_dev(inp), path=path)
    compare(f"small {path} nw={nw} init={init}", w, out, conv, S, oracle_prefill(w, inp))


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("r", [3, 8])
def test_prefill_gqa_odd_group_count(G, path, r):
    """r = 3 (the Qwen3.6-27B ratio) and r = 8 (the largest group the
    two-pass path takes) with B*H_k = 3 groups (not a multiple of 8)."""
    w = small(batch=3, num_k_heads=1, num_v_heads=r, seq_len=130, init_state=True, seed=23)
    inp = I.generate(w)
    out, conv, S = gpu_prefill(G, w, to_dev(inp), path=path)
    compare(f"gqa{r} {path}", w, out, conv, S, oracle_prefill(w, inp))


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("L", [0, 1, 2, 3, 63, 64, 65])
def test_prefill_edge_lengths(G, path, L):
    w = small(batch=1, seq_len=max(L, 1), init_state=True, seed=30 + L)
    inp = I.generate(w)
    d = to_dev(inp)
    out, conv, S = gpu_prefill(G, w, d, seq=slice(0, L), path=path)
    if L == 0:
        assert torch.equal(S, d["rec_state"]) and torch.equal(conv, d["conv_state"])
        return
    compare(f"L={L} {path}", w, out, conv, S, oracle_prefill(w, inp, seq_slice=slice(0, L)))


@pytest.mark.parametrize("path", PATHS)
def test_prefill_unaligned_split_continuation(G, path):
    """Tokens 0..99 then 100..299 from the carried state (start_pos = 100,
    first chunk partial) == the oracle over all 300 tokens."""
    w = small(seq_len=300, init_state=True, seed=24)
    inp = I.generate(w)
    d = to_dev(inp)
    o1, c1, S1 = gpu_prefill(G, w, d, seq=slice(0, 100), path=path)
    o2, c2, S2 = gpu_prefill(G, w, d, seq=slice(100, 300), start_pos=100, conv_in=c1, rec_in=S1,
                             path=path)
    ref = oracle_prefill(w, inp)
    compare(f"split@100 {path}", w, torch.cat([o1, o2], 1), c2, S2, ref)


@pytest.mark.parametrize("chunks", [1, 2, 3])
def test_prefill_segmented_workspace(G, chunks):
    """A workspace of 1, 2 or 3 chunks' worth runs the two passes segment by
    segment (state carried through rec_state_out, checkpoints included) and
    gives the single-segment result bit for bit; a workspace one byte short
    of a chunk runs the fused path."""
    w = small(seq_len=460, init_state=True, seed=29)
    inp = I.generate(w)
    d = to_dev(inp)
    c = cfg_of(G, w)
    per = G.prefill_workspace_bytes(c, 1)
    ents, nbytes = G.state_checkpoint(c, 37, 423, 128)
    bufs = [torch.zeros(nbytes, dtype=torch.uint8, device="cuda") for _ in range(2)]
    seq = slice(37, 460)
    full = gpu_prefill(G, w, d, seq=seq, start_pos=37, ckpt_interval=128, ckpt_buf=bufs[0])
    ws = torch.empty(chunks * per + 100, dtype=torch.uint8, device="cuda")
    seg = gpu_prefill(G, w, d, seq=seq, start_pos=37, ckpt_interval=128, ckpt_buf=bufs[1], workspace=ws)
    for x, y in zip(full, seg):
        assert torch.equal(x, y)
    assert torch.equal(bufs[0], bufs[1])
    fused = gpu_prefill(G, w, d, seq=seq, start_pos=37, path="fused")
    short = gpu_prefill(G, w, d, seq=seq, start_pos=37, workspace=ws[:per - 1])
    for x, y in zip(fused, short):
        assert torch.equal(x, y)


def test_prefill_paths_agree(G):
    """The two paths compute the same values in the same precision; print how
    far apart they are and hold them to a bar well inside the oracle's."""
    w = small(batch=2, seq_len=700, num_k_heads=2, num_v_heads=6, init_state=True, seed=31)
    d = to_dev(I.generate(w))
    f = gpu_prefill(G, w, d, path="fused")
    s = gpu_prefill(G, w, d, path="split")
    e_out = rel(s[0].double().cpu().numpy(), f[0].double().cpu().numpy())
    e_state = rel(s[2].double().cpu().numpy(), f[2].double().cpu().numpy())
    print(f"[paths] out rel {e_out:.3e}, state rel {e_state:.3e}, bitwise "
          f"{torch.equal(f[0], s[0]) and torch.equal(f[2], s[2])}", flush=True)
    assert torch.equal(f[1], s[1])
    assert e_out <= 1e-3 and e_state <= 1e-4


@pytest.mark.parametrize("path", PATHS)
def test_prefill_checkpoints_and_bitwise_resume(G, path):
    """Slots every 128 tokens hold the oracle's state after those positions and
    bit copies of the conv tail; resuming from a slot repeats the
    uninterrupted call bit for bit."""
    w = small(seq_len=600, init_state=True, seed=25)
    inp = I.generate(w)
    d = to_dev(inp)
    c = cfg_of(G, w)
    ents, nbytes = G.state_checkpoint(c, 0, 600, 128)
    assert [e.position for e in ents] == [128, 256, 384, 512]
    buf = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    out, conv, S = gpu_prefill(G, w, d, ckpt_interval=128, ckpt_buf=buf, path=path)
    ref = oracle_prefill(w, inp, want_ckpt=True, ckpt_interval=128)
    compare(f"ckpt run {path}", w, out, conv, S, ref)

    def slot(e):
        cv = buf[e.conv_offset:e.conv_offset + w.batch * w.conv_dim * 3 * 2].view(torch.bfloat16)
        rs = buf[e.rec_offset:e.rec_offset + w.batch * w.num_v_heads * 128 * 128 * 4].view(torch.float32)
        return cv.view(w.batch, w.conv_dim, 3), rs.view(w.batch, w.num_v_heads, 128, 128)

    for j, e in enumerate(ents):
        cv, rs = slot(e)
        assert np.array_equal(I.to_numpy_io(cv), ref["ckpt_conv"][j])
        er = rel(rs.double().cpu().numpy(), ref["ckpt_S"][j])
        assert er <= TOL_BF16_STATE, (j, er)
    # resume at slot 1 (position 256) into a fresh buffer
    cv, rs = slot(ents[1])
    buf2 = torch.zeros_like(buf)
    o2, c2, S2 = gpu_prefill(G, w, d, seq=slice(256, 600), start_pos=256, conv_in=cv.clone(),
                             rec_in=rs.clone(), ckpt_interval=128, ckpt_buf=buf2, path=path)
    assert torch.equal(o2, out[:, 256:]) and torch.equal(S2, S) and torch.equal(c2, conv)
    for e in ents[2:]:
        assert torch.equal(buf2[e.conv_offset:e.conv_offset + ents[0].rec_offset],
                           buf[e.conv_offset:e.conv_offset + ents[0].rec_offset])
        n = w.batch * w.num_v_heads * 128 * 128 * 4
        assert torch.equal(buf2[e.rec_offset:e.rec_offset + n], buf[e.rec_offset:e.rec_offset + n])


@pytest.mark.parametrize("path", PATHS)
def test_prefill_deterministic_and_in_place(G, path):
    w = small(seq_len=257, init_state=True, seed=26)
    d = to_dev(I.generate(w))
    a = gpu_prefill(G, w, d, path=path)
    b = gpu_prefill(G, w, d, path=path)
    S_in = d["rec_state"].clone()
    c = gpu_prefill(G, w, d, rec_in=S_in, rec_out=S_in, path=path)
    for x, y, z in zip(a, b, c):
        assert torch.equal(x, y) and torch.equal(x, z)


@pytest.mark.parametrize("path", PATHS)
def test_prefill_then_decode(G, path):
    """Prefill 192 tokens, then 16 decode steps from the produced state ==
    the oracle over the 208 tokens."""
    w = small(seq_len=208, init_state=True, seed=27)
    inp = I.generate(w)
    d = to_dev(inp)
    out, conv, S = gpu_prefill(G, w, d, seq=slice(0, 192), path=path)
    c = G.Config(batch=w.batch, num_k_heads=w.num_k_heads, num_v_heads=w.num_v_heads)
    outs = []
    for t in range(192, 208):
        o, conv, S = G.decode_step(c, d["qkv"][:, t].contiguous(), d["a"][:, t].contiguous(),
                                   d["b"][:, t].contiguous(), d["conv_w"], d["A_log"],
                                   d["dt_bias"], conv, S)
        outs.append(o)
    torch.cuda.synchronize()
    full = torch.cat([out, torch.stack(outs, 1)], 1)
    compare(f"prefill+decode {path}", w, full, conv, S, oracle_prefill(w, inp))


@pytest.mark.parametrize("path", PATHS)
def test_decode_stepped_equals_chunked_prefill(G, path):
    """GPU against GPU on the same tokens: 200 one-token decode steps from
    the initial states, and one chunked prefill over the 200 tokens.  The two
    evaluate the same rule in different orders (per token in fp32; per chunk
    on bf16 operands), so they agree within the bf16 bars (every 64-token
    run, every head's state); the conv tails are copies of the same inputs,
    bit for bit."""
    w = small(seq_len=200, init_state=True, seed=31)
    inp = I.generate(w)
    d = to_dev(inp)
    out_p, conv_p, S_p = gpu_prefill(G, w, d, path=path)
    c = cfg_of(G, w)
    conv, S = d["conv_state"], d["rec_state"]
    outs = []
    for t in range(w.seq_len):
        o, conv, S = G.decode_step(c, d["qkv"][:, t].contiguous(), d["a"][:, t].contiguous(),
                                   d["b"][:, t].contiguous(), d["conv_w"], d["A_log"], d["dt_bias"], conv, S)
        outs.append(o)
    torch.cuda.synchronize()
    out_d = torch.stack(outs, 1)
    assert torch.equal(conv_p, conv), "conv tails differ"
    e_run = local_rel(out_p.double().cpu().numpy(), out_d.double().cpu().numpy())
    e_out = rel(out_p.double().cpu().numpy(), out_d.double().cpu().numpy())
    e_st = state_rel_per_head(S_p.double().cpu().numpy(), S.double().cpu().numpy())
    print(f"[stepped vs chunked {path}] out rel {e_out:.3e}, worst 64-token run {e_run:.3e}, "
          f"worst head state {e_st:.3e}", flush=True)
    assert finite(out_p) and finite(out_d)
    assert e_run <= TOL_BF16_OUT and e_st <= TOL_BF16_STATE


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("stress", ["slowdecay", "extreme"])
def test_prefill_stress(G, path, stress):
    """Not among the five workloads, held to the same bars: long
    memory (decay close to 1) and gates in their tails."""
    w = small(seq_len=640, init_state=True, seed=28)
    w = I.slow_decay(w) if stress == "slowdecay" else I.extreme_gates(w)
    inp = I.generate(w)
    out, conv, S = gpu_prefill(G, w, to_dev(inp), path=path)
    compare(f"{stress} {path}", w, out, conv, S, oracle_prefill(w, inp))


@pytest.mark.parametrize("path", PATHS)
def test_prefill_orthonormal_keys_store_retrieve(G, path):
    """g = 0, beta = 1 and unit basis vectors as keys (d = 128): the state is
    a table of the last value written under each key, keys repeat inside and
    across chunks (overwrites), and the outputs read it back; held to the
    bars against the oracle."""
    w = small(seq_len=600, init_state=True, seed=41)
    inp = I.orthonormal_keys(w, I.generate(w))
    out, conv, S = gpu_prefill(G, w, to_dev(inp), path=path)
    compare(f"orthonormal {path}", w, out, conv, S, oracle_prefill(w, inp))


@pytest.mark.parametrize("path", PATHS)
def test_prefill_zero_preconv_segments(G, path):
    """Runs of all-zero pre-conv tokens (inside one chunk, across a chunk
    boundary, a whole chunk, the call's first tokens): q = k = v = 0 there,
    the l2 norm of a zero vector stays zero and the state only decays."""
    w = small(seq_len=640, init_state=True, seed=42)
    inp = I.zero_segments(I.generate(w), [(0, 5), (70, 90), (120, 200), (256, 320), (600, 640)])
    out, conv, S = gpu_prefill(G, w, to_dev(inp), path=path)
    compare(f"zero segments {path}", w, out, conv, S, oracle_prefill(w, inp))
    assert finite(out, S)


# ------------------------------------- Neumann-product diagonal solve (A/B)

@pytest.fixture
def neumann():
    """Select the Neumann-product diagonal-block solve of the two-pass path
    for one test (GDN_DIAG_SOLVE=neumann), then restore substitution."""
    old = os.environ.get("GDN_DIAG_SOLVE")
    os.environ["GDN_DIAG_SOLVE"] = "neumann"
    yield
    if old is None:
        os.environ.pop("GDN_DIAG_SOLVE", None)
    else:
        os.environ["GDN_DIAG_SOLVE"] = old


def stress_of(kind, w):
    return {"plain": lambda x: x, "slowdecay": I.slow_decay, "extreme": I.extreme_gates,
            "coincident": I.coincident_keys}[kind](w)


def gpu_prefill_solve(G, w, d, solve, path="split", precision=0):
    old = os.environ.get("GDN_DIAG_SOLVE")
    os.environ["GDN_DIAG_SOLVE"] = solve
    try:
        return gpu_prefill(G, w, d, path=path, precision=precision)
    finally:
        if old is None:
            os.environ.pop("GDN_DIAG_SOLVE", None)
        else:
            os.environ["GDN_DIAG_SOLVE"] = old


@pytest.mark.parametrize("kind", ["plain", "slowdecay", "extreme"])
def test_prefill_neumann_solve(G, kind):
    """The two-pass path with the diagonal blocks of (I + A)^-1 formed by the
    Neumann product instead of substitution, held to the same bars against
    the oracle on the plain and the stress recipes.  The distance to the
    substitution result is printed."""
    w = stress_of(kind, small(seq_len=640, init_state=True, seed=31))
    inp = I.generate(w)
    d = to_dev(inp)
    out_d, _, S_d = gpu_prefill_solve(G, w, d, "direct")
    out_n, conv_n, S_n = gpu_prefill_solve(G, w, d, "neumann")
    print(f"[neumann {kind}] vs substitution: out rel {rel(out_n.double().cpu(), out_d.double().cpu()):.3e}, "
          f"state rel {rel(S_n.double().cpu(), S_d.double().cpu()):.3e}", flush=True)
    compare(f"neumann {kind}", w, out_n, conv_n, S_n, oracle_prefill(w, inp))


# ------------------------------------------------ precise mode (hi + lo)

# Keys that nearly coincide with beta near 1 and slow decay put entries near 1
# into A, whose blocked solve then cancels heavily: the single-bf16 operands
# of the default mode (S0 in K S0 and Q S0, the coupling A_mk Delta_k, the
# diagonal product, P and Delta in P Delta) each cost about 1e-2 there (an
# fp64 model of that rounding plan gives out 1.4e-2, state 1.4e-2).  The
# precise mode takes every one of them as bf16 hi + lo (the model: out
# 1.7e-3, state 2.7e-4) and is held to the ordinary bars.

@pytest.mark.parametrize("path,solve", [("fused", "direct"), ("split", "direct"), ("split", "neumann")])
def test_prefill_coincident_keys_precise(G, path, solve):
    """Coincident keys (cosine about 0.99, beta about 1, slow decay) in the
    precise mode: the bars on the whole tensors, every 64-token run and
    every head's state, on every path and diagonal solve."""
    w = I.coincident_keys(small(seq_len=640, init_state=True, seed=31))
    inp = I.generate(w)
    out, conv, S = gpu_prefill_solve(G, w, to_dev(inp), solve, path=path, precision=G.GDN_PRECISION_HILO)
    compare(f"coincident precise {path} {solve}", w, out, conv, S, oracle_prefill(w, inp))


@pytest.mark.parametrize("path", PATHS)
def test_prefill_coincident_keys_default_reported(G, path):
    """The default mode on the same input: its distance to the oracle is
    printed beside the precise mode's (the default's single-bf16 operands
    are not held to the bars on this recipe); conv tail exact, values
    finite."""
    w = I.coincident_keys(small(seq_len=640, init_state=True, seed=31))
    inp = I.generate(w)
    ref = oracle_prefill(w, inp)
    d = to_dev(inp)
    out, conv, S = gpu_prefill(G, w, d, path=path)
    out_p, _, S_p = gpu_prefill(G, w, d, path=path, precision=G.GDN_PRECISION_HILO)
    e = [rel(x.double().cpu().numpy(), ref[k]) for x, k in ((out, "out"), (S, "S"), (out_p, "out"), (S_p, "S"))]
    print(f"[coincident {path}] default: out rel {e[0]:.3e}, state rel {e[1]:.3e}; "
          f"precise: out rel {e[2]:.3e}, state rel {e[3]:.3e}", flush=True)
    assert np.array_equal(I.to_numpy_io(conv), ref["conv_tail"])
    assert finite(out, S)


@pytest.mark.parametrize("path,nw", [("fused", None), ("split", 2), ("split", 4)])
@pytest.mark.parametrize("kind", ["plain", "slowdecay", "extreme"])
def test_prefill_precise_recipes(G, waves, path, nw, kind):
    """The precise mode on the plain and stress recipes, every state-kernel
    variant, initial states given: held to the bars."""
    waves(nw)
    w = stress_of(kind, small(seq_len=330, init_state=True, seed=33))
    inp = I.generate(w)
    out, conv, S = gpu_prefill(G, w, to_dev(inp), path=path, precision=G.GDN_PRECISION_HILO)
    compare(f"precise {kind} {path} nw={nw}", w, out, conv, S, oracle_prefill(w, inp))


def test_prefill_precise_paths_agree(G):
    """The precise mode on both paths (the fused kernel's 4-wave instance
    and the two-pass kernels), from nonzero states at an unaligned start:
    the same operations in the same order, so the same bits."""
    w = small(batch=2, seq_len=450, num_k_heads=2, num_v_heads=6, init_state=True, seed=35)
    d = to_dev(I.generate(w))
    hl = G.GDN_PRECISION_HILO
    f = gpu_prefill(G, w, d, seq=slice(19, 450), start_pos=83, path="fused", precision=hl)
    s = gpu_prefill(G, w, d, seq=slice(19, 450), start_pos=83, path="split", precision=hl)
    e_out = rel(s[0].double().cpu().numpy(), f[0].double().cpu().numpy())
    e_state = rel(s[2].double().cpu().numpy(), f[2].double().cpu().numpy())
    print(f"[precise paths] out rel {e_out:.3e}, state rel {e_state:.3e}, bitwise "
          f"{torch.equal(f[0], s[0]) and torch.equal(f[2], s[2])}", flush=True)
    assert torch.equal(f[1], s[1])
    assert torch.equal(f[0], s[0]) and torch.equal(f[2], s[2])


@pytest.mark.parametrize("path", PATHS)
def test_prefill_precise_checkpoints_and_bitwise_resume(G, path):
    """The precise mode writes the oracle's state into every checkpoint slot
    (every 128 tokens), and resuming from a slot repeats the uninterrupted
    call bit for bit."""
    w = small(seq_len=520, init_state=True, seed=36)
    inp = I.generate(w)
    d = to_dev(inp)
    hl = G.GDN_PRECISION_HILO
    c = cfg_of(G, w, hl)
    ents, nbytes = G.state_checkpoint(c, 0, 520, 128)
    buf = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    out, conv, S = gpu_prefill(G, w, d, ckpt_interval=128, ckpt_buf=buf, path=path, precision=hl)
    ref = oracle_prefill(w, inp, want_ckpt=True, ckpt_interval=128)
    compare(f"precise ckpt run {path}", w, out, conv, S, ref)
    n = w.batch * w.num_v_heads * 128 * 128 * 4
    for j, e in enumerate(ents):
        rs = buf[e.rec_offset:e.rec_offset + n].view(torch.float32).view(w.batch, w.num_v_heads, 128, 128)
        assert state_rel_per_head(rs.double().cpu().numpy(), ref["ckpt_S"][j]) <= TOL_BF16_STATE, j
    e = ents[2]   # resume at position 384
    cv = buf[e.conv_offset:e.conv_offset + w.batch * w.conv_dim * 3 * 2].view(torch.bfloat16)
    rs = buf[e.rec_offset:e.rec_offset + n].view(torch.float32)
    o2, c2, S2 = gpu_prefill(G, w, d, seq=slice(384, 520), start_pos=384,
                             conv_in=cv.view(w.batch, w.conv_dim, 3).clone(),
                             rec_in=rs.view(w.batch, w.num_v_heads, 128, 128).clone(), path=path, precision=hl)
    assert torch.equal(o2, out[:, 384:]) and torch.equal(S2, S) and torch.equal(c2, conv)


@pytest.mark.parametrize("chunks", [1, 3])
def test_prefill_precise_segmented_workspace(G, chunks):
    """Precise mode with a workspace of 1 or 3 chunks' records (the larger
    precise records): the two-pass path runs in segments and gives the
    values of the single-segment run."""
    w = small(seq_len=455, init_state=True, seed=34)
    inp = I.generate(w)
    d = to_dev(inp)
    c = cfg_of(G, w, G.GDN_PRECISION_HILO)
    per_chunk = G.prefill_workspace_bytes(c, 64)
    assert per_chunk > G.prefill_workspace_bytes(cfg_of(G, w), 64)
    ws = torch.empty(chunks * per_chunk, dtype=torch.uint8, device="cuda")
    out, conv, S = gpu_prefill(G, w, d, workspace=ws, precision=G.GDN_PRECISION_HILO)
    out1, _, S1 = gpu_prefill(G, w, d, precision=G.GDN_PRECISION_HILO)
    assert torch.equal(out, out1) and torch.equal(S, S1)
    compare(f"precise segmented {chunks}", w, out, conv, S, oracle_prefill(w, inp))


def test_workload_qwen36_prefill_16k_neumann(G, neumann):
    """The 16k workload through the two-pass path with the Neumann solve."""
    w = I.WORKLOADS[2]
    inp = I.generate(w)
    heads = [0, 23, 47]
    ref = oracle_prefill(w, inp, heads=heads)
    out, conv, S = gpu_prefill(G, w, to_dev(inp), path="split")
    compare("16k neumann", w, out, conv, S, ref, heads=heads)


# ------------------------------------------------------------ full workloads

def test_workload_qwen36_prefill_16k(G):
    """B=1, L=16384, 16/48 heads, zero state.  Sampled heads 0, 1, 2, 23, 46, 47
    (several key heads, each position in the repeat-interleave group)."""
    w = I.WORKLOADS[2]
    inp = I.generate(w)
    d = to_dev(inp)
    heads = [0, 1, 2, 23, 46, 47]
    ref = oracle_prefill(w, inp, heads=heads)
    for path in PATHS:
        out, conv, S = gpu_prefill(G, w, d, path=path)
        compare(f"16k {path}", w, out, conv, S, ref, heads=heads)


def test_workload_coder_next_prefill_4k_then_decode(G):
    """B=8, L=4096, 16/32 heads, nonzero initial state, then 64 decode steps
    continuing from the produced state.  Sampled sequences 0 and 5, heads
    0, 1, 17, 31."""
    w = I.WORKLOADS[3]
    inp = I.generate(w)
    d = to_dev(inp)
    heads, bi = [0, 1, 17, 31], [0, 5]
    full = oracle_prefill(w, inp, batch_idx=bi)
    ref = {"out": full["out"][:, :, heads], "S": full["S"][:, heads], "conv_tail": full["conv_tail"]}
    out, conv, S = gpu_prefill(G, w, d, path="fused")
    compare("4k prefill fused", w, out, conv, S, ref, heads=heads, batch_idx=bi)
    out, conv, S = gpu_prefill(G, w, d, path="split")
    compare("4k prefill split", w, out, conv, S, ref, heads=heads, batch_idx=bi)
    c = G.Config(batch=w.batch, num_k_heads=w.num_k_heads, num_v_heads=w.num_v_heads)
    outs = []
    for s in range(64):
        o, conv, S = G.decode_step(c, d["dec_qkv"][s], d["dec_a"][s], d["dec_b"][s], d["conv_w"],
                                   d["A_log"], d["dt_bias"], conv, S)
        outs.append(o)
    torch.cuda.synchronize()
    # oracle decode from the oracle's own post-prefill state (fp64, all heads of the sampled sequences)
    dref = oracle_decode(w, inp, 64, batch_idx=bi, heads=heads, conv_state=full["conv_tail"],
                         S0=full["S"])
    o = torch.stack(outs, 1)[bi][:, :, heads].double().cpu().numpy()
    e_out = rel(o, dref["out"])
    e_state = rel(S[bi][:, heads].double().cpu().numpy(), dref["S"])
    print(f"[4k decode] out rel {e_out:.3e}, state rel {e_state:.3e}", flush=True)
    assert e_out <= TOL_BF16_OUT and e_state <= TOL_BF16_STATE


@pytest.mark.timeout(600)
def test_workload_qwen36_prefill_256k_checkpoints(G):
    """B=1, L=262144, checkpoints every 4096 tokens (64 slots).  Heads 0 and
    47 against the oracle (outputs, all 64 slot states, conv tails); resume
    from three seeded-random slots is bitwise equal to the uninterrupted run."""
    w = I.WORKLOADS[4]
    print("[256k] generating inputs", flush=True)
    inp = I.generate(w)
    d = to_dev(inp)
    c = cfg_of(G, w)
    ents, nbytes = G.state_checkpoint(c, 0, w.seq_len, 4096)
    assert len(ents) == 64
    buf = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    print("[256k] GPU prefill, two-pass path", flush=True)
    out, conv, S = gpu_prefill(G, w, d, ckpt_interval=4096, ckpt_buf=buf)
    heads = [0, 1, 23, 47]
    print("[256k] oracle (4 heads)", flush=True)
    ref = oracle_prefill(w, inp, heads=heads, want_ckpt=True, ckpt_interval=4096)
    nrec = w.num_v_heads * 128 * 128 * 4

    def check_run(tag, out, conv, S, buf):
        compare(tag, w, out, conv, S, ref, heads=heads)
        worst = 0.0
        for j, e in enumerate(ents):
            rs = buf[e.rec_offset:e.rec_offset + nrec].view(torch.float32).view(1, w.num_v_heads, 128, 128)
            worst = max(worst, state_rel_per_head(rs[:, heads].double().cpu().numpy(), ref["ckpt_S"][j]))
            cv = buf[e.conv_offset:e.conv_offset + w.conv_dim * 3 * 2].view(torch.bfloat16)
            assert np.array_equal(I.to_numpy_io(cv.view(1, w.conv_dim, 3)), ref["ckpt_conv"][j])
        print(f"[{tag}] worst checkpoint state rel (per head) {worst:.3e}", flush=True)
        assert worst <= TOL_BF16_STATE

    check_run("256k two-pass", out, conv, S, buf)
    # the same call on a created stream takes the overlapped prep (head chunks
    # first, the rest beside the state kernel): bit for bit the serial run,
    # checkpoint slots included
    print("[256k] GPU prefill, two-pass path with the overlapped prep (side stream)", flush=True)
    buf_o = torch.zeros_like(buf)
    ws = torch.zeros(G.prefill_workspace_bytes(c, w.seq_len), dtype=torch.uint8, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        out_o, conv_o, S_o = gpu_prefill(G, w, d, ckpt_interval=4096, ckpt_buf=buf_o, workspace=ws)
    torch.cuda.synchronize()
    n = w.seq_len // 64
    per = G.prefill_workspace_bytes(c, 1)
    flags = ws[n * per:n * per + 8 * w.num_k_heads * n].view(torch.int64).view(w.num_k_heads, n)
    assert bool((flags[:, n - 1] != 0).all()), "the tail prep did not publish the last chunk"
    assert torch.equal(out_o, out) and torch.equal(conv_o, conv) and torch.equal(S_o, S)
    assert torch.equal(buf_o, buf), "checkpoint slots differ between the overlapped and the serial run"
    del out_o, conv_o, S_o, buf_o, ws, flags
    print("[256k] GPU prefill, fused path", flush=True)
    buf_f = torch.zeros_like(buf)
    out_f, conv_f, S_f = gpu_prefill(G, w, d, ckpt_interval=4096, ckpt_buf=buf_f, path="fused")
    check_run("256k fused", out_f, conv_f, S_f, buf_f)
    # all 48 heads: the two paths against each other, run by run, within the bars
    B, L, H, dv = out.shape
    diff = (out_f.float() - out.float()).square().view(B, L // 64, 64, H, dv).sum((2, 4))
    ref2 = out.float().square().view(B, L // 64, 64, H, dv).sum((2, 4))
    e_paths = float((diff / ref2.clamp_min(1e-30)).sqrt().max())
    del diff, ref2
    s_paths = state_rel_per_head(S_f.double().cpu().numpy(), S.double().cpu().numpy())
    print(f"[256k] fused vs two-pass, all heads: worst 64-token run {e_paths:.3e}, "
          f"worst head state {s_paths:.3e}", flush=True)
    assert e_paths <= TOL_BF16_OUT and s_paths <= TOL_BF16_STATE
    del out_f, conv_f, S_f, buf_f
    rng = np.random.default_rng(2024)
    for j in sorted(rng.choice(63, size=3, replace=False)):
        e = ents[j]
        p = e.position
        cv = buf[e.conv_offset:e.conv_offset + w.conv_dim * 3 * 2].view(torch.bfloat16).view(1, w.conv_dim, 3)
        rs = buf[e.rec_offset:e.rec_offset + nrec].view(torch.float32).view(1, w.num_v_heads, 128, 128)
        o2, c2, S2 = gpu_prefill(G, w, d, seq=slice(p, None), start_pos=p, conv_in=cv.clone(),
                                 rec_in=rs.clone())
        print(f"[256k] resume from slot {j} (position {p})", flush=True)
        assert torch.equal(o2, out[:, p:]) and torch.equal(S2, S) and torch.equal(c2, conv)
