"""GPU parity of the one-token recurrent decode step (gdn_decode_step) with the
fp64 oracle, through the C ABI.

The oracle of S steps is the per-token rule over those S tokens as one call;
the oracle's own split-anywhere test pins that this equals S single steps.
"""
import numpy as np
import pytest
import torch

from linear_attention_recurrence_causal_amd import inputs as I
from tests.helpers import finite, oracle_decode, rel, to_dev, tols

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


def run_steps(G, w, d, steps, in_place=True, null_state=False):
    """`steps` decode calls; conv state ping-pongs, recurrent state in place."""
    c = cfg_of(G, w)
    B, Hv = w.batch, w.num_v_heads
    S = (d["rec_state"].clone() if d["rec_state"] is not None
         else torch.zeros(B, Hv, w.head_k_dim, w.head_v_dim, device="cuda"))
    cs0 = (d["conv_state"].clone() if d["conv_state"] is not None
           else torch.zeros(B, w.conv_dim, 3, dtype=w.io_dtype, device="cuda"))
    cs = [cs0, torch.empty_like(cs0)]
    outs = torch.empty(steps, B, Hv, w.head_v_dim, dtype=w.io_dtype, device="cuda")
    for s in range(steps):
        cin = None if (null_state and s == 0 and d["conv_state"] is None) else cs[s % 2]
        rin = None if (null_state and s == 0 and d["rec_state"] is None) else S
        Sout = S if in_place else torch.empty_like(S)
        G.decode_step(c, d["dec_qkv"][s], d["dec_a"][s], d["dec_b"][s], d["conv_w"], d["A_log"],
                      d["dt_bias"], cin, rin, out=outs[s], conv_state_out=cs[(s + 1) % 2],
                      rec_state_out=Sout)
        S = Sout
    torch.cuda.synchronize()
    return outs, cs[steps % 2], S


def check_against_oracle(w, inp, outs, conv, S, batch_idx=None):
    steps = outs.shape[0]
    ref = oracle_decode(w, inp, steps, batch_idx=batch_idx)
    bi = list(range(w.batch)) if batch_idx is None else list(batch_idx)
    o = outs[:, bi].transpose(0, 1).double().cpu().numpy()
    t_out, t_state = tols(w)
    e_out = rel(o, ref["out"])
    e_state = rel(S[bi].double().cpu().numpy(), ref["S"])
    print(f"[decode {w.name}] steps={steps} out rel {e_out:.3e} (bar {t_out}), "
          f"state rel {e_state:.3e} (bar {t_state})", flush=True)
    assert e_out <= t_out
    assert e_state <= t_state
    assert np.array_equal(I.to_numpy_io(conv[bi]), ref["conv_tail"])
    assert finite(outs, S)


def test_decode_tiny_f32_64_steps(G):
    """Tiny fp32 workload (B=1, 2 key / 4 value heads, d=32, zero state),
    the recurrent path for 64 tokens."""
    w = I.WORKLOADS[0]
    inp = I.generate(w)
    outs, conv, S = run_steps(G, w, to_dev(inp), 64)
    check_against_oracle(w, inp, outs, conv, S)


def test_decode_qwen36_b32_256_steps(G):
    """Qwen3.6-27B-shaped decode: B=32, 16/48 heads, d=128, bf16 io, fp32
    state ~N(0, 0.05), 256 steps.  All 32 sequences run on the GPU; the
    oracle checks sequences 0, 13 and 31 over all heads and all steps."""
    w = I.WORKLOADS[1]
    inp = I.generate(w)
    outs, conv, S = run_steps(G, w, to_dev(inp), 256)
    check_against_oracle(w, inp, outs, conv, S, batch_idx=[0, 13, 31])


@pytest.mark.parametrize("dk,dv,io", [(64, 32, "bf16"), (128, 64, "f32"), (32, 128, "bf16"),
                                      (128, 128, "f32")])
def test_decode_head_dims(G, dk, dv, io):
    w = I.Workload("dims", batch=3, seq_len=0, num_k_heads=2, num_v_heads=6, head_k_dim=dk,
                   head_v_dim=dv, io=io, decode_steps=20, init_state=True, seed=77)
    inp = I.generate(w)
    outs, conv, S = run_steps(G, w, to_dev(inp), 20)
    check_against_oracle(w, inp, outs, conv, S)


def test_decode_in_place_null_state_and_determinism(G):
    w = I.Workload("np", batch=2, seq_len=0, num_k_heads=2, num_v_heads=4, decode_steps=8,
                   seed=78)
    inp = I.generate(w)
    d = to_dev(inp)
    a = run_steps(G, w, d, 8, in_place=True)
    b = run_steps(G, w, d, 8, in_place=False)
    c = run_steps(G, w, d, 8, in_place=True, null_state=True)   # NULL = zeros
    for x, y, z in zip(a, b, c):
        assert torch.equal(x, y) and torch.equal(x, z)
    check_against_oracle(w, inp, *a)
