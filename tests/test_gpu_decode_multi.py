"""GPU parity of the multi-token decode step (gdn_decode_multi), through the
C ABI: T tokens per call equal T one-token calls (gdn_decode_step) bit for
bit -- outputs, final states, conv tails and every per-token snapshot -- and
match the fp64 oracle, whose checkpoints at interval 1 give the state after
each token.
"""
import numpy as np
import pytest
import torch

from linear_attention_recurrence_causal_amd import inputs as I
from tests.helpers import dims, finite, np_io, rel, to_dev, tols

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def G():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from linear_attention_recurrence_causal_amd import gdn
    return gdn


def cfg_of(G, w):
    return G.Config(batch=w.batch, num_k_heads=w.num_k_heads, num_v_heads=w.num_v_heads,
                    head_k_dim=w.head_k_dim, head_v_dim=w.head_v_dim,
                    io_dtype=G.GDN_F32 if w.io == "f32" else G.GDN_BF16)


def tokens(d, t0, T, key):
    """Decode inputs of tokens t0 .. t0 + T - 1 as [B, T, ...]."""
    return d[key][t0:t0 + T].transpose(0, 1).contiguous()


def init_states(w, d):
    B, Hv = w.batch, w.num_v_heads
    S = (d["rec_state"].clone() if d["rec_state"] is not None
         else torch.zeros(B, Hv, w.head_k_dim, w.head_v_dim, device="cuda"))
    cs = (d["conv_state"].clone() if d["conv_state"] is not None
          else torch.zeros(B, w.conv_dim, 3, dtype=w.io_dtype, device="cuda"))
    return S, cs


def single_steps(G, w, d, t0, T, S, cs):
    """T one-token calls from (S, cs); returns outputs [B, T, ...], the state
    and conv tail after every token."""
    c = cfg_of(G, w)
    outs, states, convs = [], [], []
    for t in range(t0, t0 + T):
        o, cs, S = G.decode_step(c, d["dec_qkv"][t], d["dec_a"][t], d["dec_b"][t], d["conv_w"],
                                 d["A_log"], d["dt_bias"], cs, S)
        outs.append(o)
        states.append(S)
        convs.append(cs)
    torch.cuda.synchronize()
    return torch.stack(outs, 1), states, convs


def multi(G, w, d, t0, T, S, cs, snapshots=True):
    c = cfg_of(G, w)
    out, cso, So, rs, csn = G.decode_multi(c, tokens(d, t0, T, "dec_qkv"), tokens(d, t0, T, "dec_a"),
                                           tokens(d, t0, T, "dec_b"), d["conv_w"], d["A_log"],
                                           d["dt_bias"], cs, S, snapshots=snapshots)
    torch.cuda.synchronize()
    return out, cso, So, rs, csn


WORKLOADS = [
    I.Workload("tiny_f32", batch=1, seq_len=0, num_k_heads=2, num_v_heads=4, head_k_dim=32,
               head_v_dim=32, io="f32", decode_steps=16, seed=90),
    I.Workload("qwen_b4", batch=4, seq_len=0, num_k_heads=16, num_v_heads=48, decode_steps=16,
               init_state=True, seed=91),
    I.Workload("dims_64_32", batch=3, seq_len=0, num_k_heads=2, num_v_heads=6, head_k_dim=64,
               head_v_dim=32, decode_steps=16, init_state=True, seed=92),
]


@pytest.mark.parametrize("w", WORKLOADS, ids=lambda w: w.name)
@pytest.mark.parametrize("T", [1, 2, 5, 8])
def test_multi_equals_single_steps_bitwise(G, w, T):
    d = to_dev(I.generate(w))
    S0, cs0 = init_states(w, d)
    out1, states, convs = single_steps(G, w, d, 0, T, S0.clone(), cs0.clone())
    outm, csm, Sm, rs, csn = multi(G, w, d, 0, T, S0.clone(), cs0.clone())
    assert torch.equal(outm, out1)
    assert torch.equal(Sm, states[-1]) and torch.equal(csm, convs[-1])
    for t in range(T):
        assert torch.equal(rs[t], states[t]), t
        assert torch.equal(csn[t], convs[t]), t
    # without snapshots the same results
    outn, csn2, Sn, rs2, cs2 = multi(G, w, d, 0, T, S0.clone(), cs0.clone(), snapshots=False)
    assert rs2 is None and cs2 is None
    assert torch.equal(outn, outm) and torch.equal(Sn, Sm) and torch.equal(csn2, csm)
    print(f"[multi {w.name} T={T}] bitwise equal to {T} single steps", flush=True)


def test_multi_chained_calls_and_null_state(G):
    """Calls of 3, 8 and 5 tokens back to back == 16 single steps; NULL
    states are zeros."""
    w = I.Workload("chain", batch=2, seq_len=0, num_k_heads=4, num_v_heads=8, decode_steps=16, seed=93)
    d = to_dev(I.generate(w))
    S0, cs0 = init_states(w, d)
    out1, states, convs = single_steps(G, w, d, 0, 16, S0.clone(), cs0.clone())
    c = cfg_of(G, w)
    S, cs, outs, t0 = None, None, [], 0     # NULL states on the first call
    for T in (3, 8, 5):
        o, cs, S, _, _ = G.decode_multi(c, tokens(d, t0, T, "dec_qkv"), tokens(d, t0, T, "dec_a"),
                                        tokens(d, t0, T, "dec_b"), d["conv_w"], d["A_log"], d["dt_bias"],
                                        cs, S)
        outs.append(o)
        t0 += T
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(outs, 1), out1)
    assert torch.equal(S, states[-1]) and torch.equal(cs, convs[-1])


@pytest.mark.parametrize("w", WORKLOADS[:2], ids=lambda w: w.name)
def test_multi_matches_oracle_per_token(G, w):
    """T = 8: outputs, final state and every snapshot against the fp64 oracle
    (the state after each token from its checkpoints at interval 1)."""
    from oracle import oracle as O
    T = 8
    inp = I.generate(w)
    d = to_dev(inp)
    S0, cs0 = init_states(w, d)
    out, cso, So, rs, csn = multi(G, w, d, 0, T, S0, cs0)
    qkv = np_io(inp["dec_qkv"][:T].transpose(0, 1).contiguous())
    a = np_io(inp["dec_a"][:T].transpose(0, 1).contiguous())
    b = np_io(inp["dec_b"][:T].transpose(0, 1).contiguous())
    cs_np = np_io(inp["conv_state"]) if inp["conv_state"] is not None else None
    S_np = inp["rec_state"].double().numpy() if inp["rec_state"] is not None else None
    dd = dims(w, seq_len=T, ckpt_interval=1)
    ref = O.layer(dd, qkv, a, b, np_io(inp["conv_w"]), inp["A_log"].numpy(), inp["dt_bias"].numpy(),
                  cs_np, S_np, want_ckpt=True)
    tail, ck = O.conv_tail(dd, qkv, cs_np, want_ckpt=True)
    t_out, t_state = tols(w)
    e_out = rel(out.double().cpu().numpy(), ref["out"])
    e_state = rel(So.double().cpu().numpy(), ref["S"])
    e_snap = max(rel(rs[t].double().cpu().numpy(), ref["ckpt_S"][t]) for t in range(T))
    print(f"[multi {w.name} T={T}] out rel {e_out:.3e} (bar {t_out}), state rel {e_state:.3e}, "
          f"worst snapshot {e_snap:.3e} (bar {t_state})", flush=True)
    assert e_out <= t_out and e_state <= t_state and e_snap <= t_state
    assert np.array_equal(I.to_numpy_io(cso), tail)
    for t in range(T):
        assert np.array_equal(I.to_numpy_io(csn[t]), ck[t]), t
    assert finite(out, So, rs)


def test_multi_snapshots_beyond_4gib(G):
    """One state snapshot of more than 4 GiB (B * H_v = 65,568 heads of
    128 x 128): every head's snapshot slice is addressed from its own base,
    so the heads at the end of the snapshot land where they belong.  Two
    tokens in one call equal two one-token calls bit for bit, snapshots
    included (checked on every head)."""
    B, Hk, Hv, d, T = 1366, 16, 48, 128, 2
    assert B * Hv * d * d * 4 > 4 * 2 ** 30
    c = G.Config(batch=B, num_k_heads=Hk, num_v_heads=Hv, head_k_dim=d, head_v_dim=d, io_dtype=G.GDN_BF16)
    gen = torch.Generator(device="cuda").manual_seed(4242)
    bf = torch.bfloat16
    qkv = torch.randn(B, T, c.conv_dim, device="cuda", generator=gen).to(bf)
    a = torch.randn(B, T, Hv, device="cuda", generator=gen).to(bf)
    b = torch.randn(B, T, Hv, device="cuda", generator=gen).to(bf)
    conv_w = (0.5 * torch.randn(c.conv_dim, 4, device="cuda", generator=gen)).to(bf)
    A_log = torch.log(1 + 15 * torch.rand(Hv, device="cuda", generator=gen))
    dt_bias = 0.1 * torch.randn(Hv, device="cuda", generator=gen)
    cs = torch.randn(B, c.conv_dim, 3, device="cuda", generator=gen).to(bf)
    S0 = 0.05 * torch.randn(B, Hv, d, d, device="cuda", generator=gen)
    print(f"[multi >4GiB] B={B} H_v={Hv}: snapshot {B * Hv * d * d * 4 / 2 ** 30:.3f} GiB per token",
          flush=True)
    out, cso, So, rs, csn = G.decode_multi(c, qkv, a, b, conv_w, A_log, dt_bias, cs, S0, snapshots=True)
    o1, cs1, S1 = G.decode_step(c, qkv[:, 0].contiguous(), a[:, 0].contiguous(), b[:, 0].contiguous(),
                                conv_w, A_log, dt_bias, cs, S0)
    assert torch.equal(rs[0], S1) and torch.equal(csn[0], cs1)
    del S0
    o2, cs2, S2 = G.decode_step(c, qkv[:, 1].contiguous(), a[:, 1].contiguous(), b[:, 1].contiguous(),
                                conv_w, A_log, dt_bias, cs1, S1)
    assert torch.equal(rs[1], S2) and torch.equal(So, S2) and torch.equal(csn[1], cs2)
    assert torch.equal(out[:, 0], o1) and torch.equal(out[:, 1], o2)
    torch.cuda.synchronize()
