"""GPU parity of the output gate ("Output": RMSNormGated of the core output
with z), through the C ABI: the standalone gdn_output_gate against the fp64
oracle on given o, z, w (every supported d_v, both io dtypes, ragged row
counts, in place, zero rows, the full prefill output shape sampled), after a
prefill end to end, and the gate fused into the decode step
(gdn_decode_gated) against the oracle per token and bitwise against the
ungated step for out, states and snapshots.
"""
import os

import numpy as np
import pytest
import torch

from linear_attention_recurrence_causal_amd import inputs as I
from tests.helpers import (finite, io_to_f64, np_io, oracle_decode, oracle_prefill, rel, to_dev,
                           tols)

pytestmark = pytest.mark.gpu

EPS = 1e-6


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


def oracle_gate(o, z, w_):
    """fp64 oracle on io tensors (or fp64 arrays for o)."""
    from oracle import oracle as O
    o64 = o if isinstance(o, np.ndarray) and o.dtype == np.float64 else io_to_f64(np_io(o.cpu()))
    return O.output_gate(o64, io_to_f64(np_io(z.cpu())), io_to_f64(np_io(w_.cpu())), EPS)


def gate_case(io, dv, n_tok, Hv=3, seed=0):
    return I.Workload("gate", batch=1, seq_len=0, num_k_heads=1, num_v_heads=Hv, head_k_dim=dv,
                      head_v_dim=dv, io=io, seed=seed)


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("dv", [32, 64, 128])
@pytest.mark.parametrize("n_tok", [1, 37, 301])
def test_output_gate_small(G, io, dv, n_tok):
    """Row counts n_tok * 3 that leave a ragged last workgroup; o with rows of
    very different scale."""
    w = gate_case(io, dv, n_tok, seed=dv + n_tok)
    gen = torch.Generator().manual_seed(dv * 1000 + n_tok)
    o = (torch.randn((n_tok, w.num_v_heads, dv), generator=gen)
         * torch.exp(2 * torch.randn((n_tok, w.num_v_heads, 1), generator=gen))).to(w.io_dtype)
    gi = I.gate_inputs(w, (n_tok,))
    od, zd, wd = o.cuda(), gi["z"].cuda(), gi["norm_w"].cuda()
    y = G.output_gate(cfg_of(G, w), od, zd, wd, EPS)
    torch.cuda.synchronize()
    ref = oracle_gate(o, gi["z"], gi["norm_w"])
    e = rel(y.double().cpu().numpy(), ref)
    bar = 1e-4 if io == "f32" else 1e-2
    print(f"[gate {io} dv={dv} rows={n_tok * 3}] rel {e:.3e} (bar {bar})", flush=True)
    assert e <= bar and finite(y)
    if io == "bf16":
        # each element within one bf16 step of the oracle rounded to bf16
        want = torch.from_numpy(ref).to(torch.bfloat16).view(torch.int16).int()
        got = y.cpu().view(torch.int16).int()
        assert int((want - got).abs().max()) <= 1


def test_output_gate_in_place_and_edges(G):
    w = gate_case("bf16", 128, 50, Hv=4, seed=3)
    c = cfg_of(G, w)
    gen = torch.Generator().manual_seed(3)
    o = torch.randn((50, 4, 128), generator=gen).to(torch.bfloat16)
    o[7, 2] = 0.0   # a zero row gives zeros (eps > 0)
    gi = I.gate_inputs(w, (50,))
    od, zd, wd = o.cuda(), gi["z"].cuda(), gi["norm_w"].cuda()
    y = G.output_gate(c, od, zd, wd, EPS)
    y_o = G.output_gate(c, od.clone(), zd, wd, EPS, y=None)
    oo = od.clone()
    G.output_gate(c, oo, zd, wd, EPS, y=oo)       # in place over o
    zz = zd.clone()
    G.output_gate(c, od, zz, wd, EPS, y=zz)       # in place over z
    empty = torch.empty((0, 4, 128), dtype=torch.bfloat16, device="cuda")
    G.output_gate(c, empty, empty.clone(), wd, EPS)   # no rows: nothing to do
    torch.cuda.synchronize()
    assert torch.equal(y, y_o) and torch.equal(y, oo) and torch.equal(y, zz)
    assert bool((y[7, 2] == 0).all()) and finite(y)


def test_output_gate_prefill_output_shape(G):
    """The 16k prefill's output shape [16384, 48, 128] bf16 in one call;
    every 97th row against the oracle."""
    w = I.WORKLOADS[2]
    gen = torch.Generator().manual_seed(77)
    o = torch.randn((w.seq_len, w.num_v_heads, w.head_v_dim), generator=gen).to(torch.bfloat16)
    gi = I.gate_inputs(w, (w.seq_len,))
    y = G.output_gate(cfg_of(G, w), o.cuda(), gi["z"].cuda(), gi["norm_w"].cuda(), EPS)
    torch.cuda.synchronize()
    rows = slice(0, None, 97)
    o2 = o.reshape(-1, w.head_v_dim)[rows]
    z2 = gi["z"].reshape(-1, w.head_v_dim)[rows]
    ref = oracle_gate(o2, z2, gi["norm_w"])
    e = rel(y.reshape(-1, w.head_v_dim)[rows].double().cpu().numpy(), ref)
    print(f"[gate 16k shape] rel {e:.3e}", flush=True)
    assert e <= 1e-2 and finite(y)


def test_output_gate_after_prefill(G):
    """Prefill (two-pass path) then the gate, against the oracle's prefill
    output gated in fp64."""
    w = I.Workload("small", batch=2, seq_len=200, num_k_heads=2, num_v_heads=4, init_state=True,
                   seed=41)
    inp = I.generate(w)
    d = to_dev(inp)
    c = cfg_of(G, w)
    ws = torch.empty(G.prefill_workspace_bytes(c, w.seq_len), dtype=torch.uint8, device="cuda")
    out, _, _ = G.prefill_chunked(c, d["qkv"], d["a"], d["b"], d["conv_w"], d["A_log"], d["dt_bias"],
                                  d["conv_state"], d["rec_state"], workspace=ws)
    gi = I.gate_inputs(w, (w.batch, w.seq_len))
    y = G.output_gate(c, out, gi["z"].cuda(), gi["norm_w"].cuda(), EPS)
    torch.cuda.synchronize()
    ref = oracle_gate(oracle_prefill(w, inp)["out"], gi["z"], gi["norm_w"])
    e = rel(y.double().cpu().numpy(), ref)
    print(f"[prefill + gate] rel {e:.3e}", flush=True)
    assert e <= tols(w)[0] and finite(y)


# ------------------------------------------------------------ fused in decode

DECODE_WORKLOADS = [
    I.Workload("tiny_f32", batch=1, seq_len=0, num_k_heads=2, num_v_heads=4, head_k_dim=32,
               head_v_dim=32, io="f32", decode_steps=8, seed=95),
    I.Workload("qwen_b32", batch=32, seq_len=0, num_k_heads=16, num_v_heads=48, decode_steps=8,
               init_state=True, seed=96),
    I.Workload("dims_64_64", batch=3, seq_len=0, num_k_heads=2, num_v_heads=6, head_k_dim=64,
               head_v_dim=64, decode_steps=8, init_state=True, seed=97),
]


def tokens(d, T, key):
    return d[key][:T].transpose(0, 1).contiguous()


def init_states(w, d):
    S = (d["rec_state"].clone() if d["rec_state"] is not None
         else torch.zeros(w.batch, w.num_v_heads, w.head_k_dim, w.head_v_dim, device="cuda"))
    cs = (d["conv_state"].clone() if d["conv_state"] is not None
          else torch.zeros(w.batch, w.conv_dim, 3, dtype=w.io_dtype, device="cuda"))
    return S, cs


@pytest.mark.parametrize("w", DECODE_WORKLOADS, ids=lambda w: w.name)
@pytest.mark.parametrize("T", [1, 4])
def test_decode_gated(G, w, T):
    inp = I.generate(w)
    d = to_dev(inp)
    c = cfg_of(G, w)
    gi = I.gate_inputs(w, (w.batch, T))
    z, nw = gi["z"].cuda(), gi["norm_w"].cuda()
    S, cs = init_states(w, d)
    snaps = T > 1
    y, out, cso, So, rs, csn = G.decode_gated(c, tokens(d, T, "dec_qkv"), tokens(d, T, "dec_a"),
                                              tokens(d, T, "dec_b"), d["conv_w"], d["A_log"],
                                              d["dt_bias"], z, nw, cs, S, eps=EPS, want_out=True,
                                              snapshots=snaps)
    y_only = G.decode_gated(c, tokens(d, T, "dec_qkv"), tokens(d, T, "dec_a"), tokens(d, T, "dec_b"),
                            d["conv_w"], d["A_log"], d["dt_bias"], z, nw, cs, S, eps=EPS)[0]
    # the ungated step with the same column split
    old = os.environ.get("GDN_DECODE_COLS")
    os.environ["GDN_DECODE_COLS"] = str(w.head_v_dim)
    try:
        out_u, cs_u, S_u, rs_u, csn_u = G.decode_multi(c, tokens(d, T, "dec_qkv"), tokens(d, T, "dec_a"),
                                                       tokens(d, T, "dec_b"), d["conv_w"], d["A_log"],
                                                       d["dt_bias"], cs, S, snapshots=snaps)
    finally:
        if old is None:
            os.environ.pop("GDN_DECODE_COLS", None)
        else:
            os.environ["GDN_DECODE_COLS"] = old
    torch.cuda.synchronize()
    assert torch.equal(out, out_u) and torch.equal(So, S_u) and torch.equal(cso, cs_u)
    if snaps:
        assert torch.equal(rs, rs_u) and torch.equal(csn, csn_u)
    assert torch.equal(y, y_only)
    ref = oracle_decode(w, inp, T)
    ref_y = oracle_gate(ref["out"], gi["z"], gi["norm_w"])
    e_y, e_o = rel(y.double().cpu().numpy(), ref_y), rel(out.double().cpu().numpy(), ref["out"])
    t_out, _ = tols(w)
    print(f"[decode gated {w.name} T={T}] y rel {e_y:.3e}, out rel {e_o:.3e} (bar {t_out})", flush=True)
    assert e_y <= t_out and e_o <= t_out and finite(y)
