"""GPU parity of the varlen prefill (gdn_prefill_varlen), through the C ABI:
sequences of different lengths and start positions packed along the token
axis give, sequence by sequence, bit for bit what gdn_prefill_chunked gives
for that sequence alone -- outputs, final states, conv tails and checkpoint
slots -- with the whole call in one segment or in segments of one chunk,
across several groups of 64 sequences, and match the fp64 oracle.
"""
import numpy as np
import pytest
import torch

from linear_attention_recurrence_causal_amd import inputs as I
from tests.helpers import finite, oracle_prefill, rel, tols

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def G():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from linear_attention_recurrence_causal_amd import gdn
    return gdn


def packed_case(lens, starts, Hk=2, Hv=4, seed=60, init=True):
    """Inputs of a B = len(lens) workload of max(lens) tokens; sequence i uses
    its first lens[i] tokens.  Returns the workload, its inputs and the
    packed qkv, a, b."""
    w = I.Workload("varlen", batch=len(lens), seq_len=max(max(lens), 1), num_k_heads=Hk, num_v_heads=Hv,
                   init_state=init, seed=seed)
    inp = I.generate(w)
    qkv = torch.cat([inp["qkv"][i, :n] for i, n in enumerate(lens)])
    a = torch.cat([inp["a"][i, :n] for i, n in enumerate(lens)])
    b = torch.cat([inp["b"][i, :n] for i, n in enumerate(lens)])
    return w, inp, qkv, a, b


def cu_of(lens):
    return [0] + list(np.cumsum(lens))


def run_varlen(G, w, inp, qkv, a, b, lens, starts, ckpt_interval=0, workspace="auto", precision=0):
    c = G.Config(batch=w.batch, num_k_heads=w.num_k_heads, num_v_heads=w.num_v_heads, precision=precision)
    ck = None
    if ckpt_interval:
        need = max(G.state_checkpoint(c, s, n, ckpt_interval)[1] for s, n in zip(starts, lens))
        ck = torch.full((max(need, 256),), 0x5A, dtype=torch.uint8, device="cuda")
    d = lambda t: None if t is None else t.cuda()
    out, conv, S = G.prefill_varlen(c, cu_of(lens), starts, qkv.cuda(), a.cuda(), b.cuda(), d(inp["conv_w"]),
                                    d(inp["A_log"]), d(inp["dt_bias"]), d(inp["conv_state"]),
                                    d(inp["rec_state"]), ckpt_interval=ckpt_interval, ckpt_buf=ck,
                                    workspace=workspace)
    torch.cuda.synchronize()
    return c, out, conv, S, ck


def run_single(G, w, inp, i, n, start, ckpt_interval=0, precision=0):
    """Sequence i alone through gdn_prefill_chunked (two-pass path)."""
    c = G.Config(batch=1, num_k_heads=w.num_k_heads, num_v_heads=w.num_v_heads, precision=precision)
    sl = lambda t: None if t is None else t[i:i + 1].contiguous().cuda()
    ck = None
    if ckpt_interval:
        need = G.state_checkpoint(c, start, n, ckpt_interval)[1]
        ck = torch.zeros((max(need, 256),), dtype=torch.uint8, device="cuda")
    out, conv, S = G.prefill_chunked(c, inp["qkv"][i:i + 1, :n].contiguous().cuda(),
                                     inp["a"][i:i + 1, :n].contiguous().cuda(),
                                     inp["b"][i:i + 1, :n].contiguous().cuda(), inp["conv_w"].cuda(),
                                     inp["A_log"].cuda(), inp["dt_bias"].cuda(), sl(inp["conv_state"]),
                                     sl(inp["rec_state"]), start_pos=start, ckpt_interval=ckpt_interval,
                                     ckpt_buf=ck)
    torch.cuda.synchronize()
    return out[0], conv[0], S[0], ck


def check_against_singles(G, w, inp, lens, starts, out, conv, S, ck=None, ckpt_interval=0, cfg=None, precision=0):
    cu = cu_of(lens)
    for i, (n, st) in enumerate(zip(lens, starts)):
        o1, c1, S1, ck1 = run_single(G, w, inp, i, n, st, ckpt_interval, precision)
        assert torch.equal(out[cu[i]:cu[i + 1]], o1), f"out of sequence {i}"
        assert torch.equal(conv[i], c1), f"conv tail of sequence {i}"
        assert torch.equal(S[i], S1), f"state of sequence {i}"
        if ckpt_interval:
            c1cfg = G.Config(batch=1, num_k_heads=w.num_k_heads, num_v_heads=w.num_v_heads)
            ents1, _ = G.state_checkpoint(c1cfg, st, n, ckpt_interval)
            for e1 in ents1:
                e = G.ckpt_lookup(cfg, ckpt_interval, e1.position, i)
                assert e.slot == e1.slot
                cb = conv[i].numel() * 2
                rb = S[i].numel() * 4
                assert torch.equal(ck[e.conv_offset:e.conv_offset + cb], ck1[e1.conv_offset:e1.conv_offset + cb])
                assert torch.equal(ck[e.rec_offset:e.rec_offset + rb], ck1[e1.rec_offset:e1.rec_offset + rb])


LENS = [200, 0, 1, 64, 130, 700, 63, 65]
STARTS = [0, 17, 63, 64, 5, 128, 1, 4096]


@pytest.mark.parametrize("segmented", [False, True])
def test_varlen_equals_single_calls(G, segmented):
    """Eight sequences: empty, one token, exactly one chunk, ragged both
    ends, unaligned starts; whole call in one segment or one chunk per
    sequence per segment."""
    w, inp, qkv, a, b = packed_case(LENS, STARTS)
    ws = "auto"
    if segmented:
        c = G.Config(batch=w.batch, num_k_heads=w.num_k_heads, num_v_heads=w.num_v_heads)
        ws = torch.empty(G.prefill_varlen_workspace_bytes(c, [0, 1] + [1] * 7, [0] * 8) // 1,
                         dtype=torch.uint8, device="cuda")
        assert ws.numel() == 8 * (2 * 32768 + 4 * 13568)
    c, out, conv, S, _ = run_varlen(G, w, inp, qkv, a, b, LENS, STARTS, workspace=ws)
    check_against_singles(G, w, inp, LENS, STARTS, out, conv, S)
    assert finite(out, S)


@pytest.mark.parametrize("segmented", [False, True])
def test_varlen_precise_equals_single_calls(G, segmented):
    """The precise mode (larger value records) through the varlen entry:
    bitwise equal to precise single calls, in one segment or in segments of
    one chunk per sequence."""
    w, inp, qkv, a, b = packed_case(LENS, STARTS, seed=64)
    ws = "auto"
    if segmented:
        c = G.Config(batch=w.batch, num_k_heads=w.num_k_heads, num_v_heads=w.num_v_heads,
                     precision=G.GDN_PRECISION_HILO)
        ws = torch.empty(G.prefill_varlen_workspace_bytes(c, [0, 1] + [1] * 7, [0] * 8),
                         dtype=torch.uint8, device="cuda")
        assert ws.numel() == 8 * (2 * 32768 + 4 * 26624)
    c, out, conv, S, _ = run_varlen(G, w, inp, qkv, a, b, LENS, STARTS, workspace=ws,
                                    precision=G.GDN_PRECISION_HILO)
    check_against_singles(G, w, inp, LENS, STARTS, out, conv, S, precision=G.GDN_PRECISION_HILO)
    assert finite(out, S)


def test_varlen_checkpoints(G):
    """Checkpoints every 64 tokens: every slot a sequence writes holds what
    its single call writes, and slots a sequence does not reach keep the
    fill pattern."""
    lens, starts = [300, 70, 0, 130], [0, 60, 64, 130]
    w, inp, qkv, a, b = packed_case(lens, starts, seed=61)
    c, out, conv, S, ck = run_varlen(G, w, inp, qkv, a, b, lens, starts, ckpt_interval=64)
    check_against_singles(G, w, inp, lens, starts, out, conv, S, ck, 64, cfg=c)
    # sequence 1 (positions 60..130) writes slots 0 (pos 64) and 1 (pos 128) only
    e = G.ckpt_lookup(c, 64, 256, 1)   # slot 3 (position 256) was not reached by it
    nb = S[1].numel() * 4
    assert bool((ck[e.rec_offset:e.rec_offset + nb] == 0x5A).all())


def test_varlen_many_groups(G):
    """70 sequences (two groups of the kernels' 64) of 0..150 tokens."""
    rng = np.random.default_rng(62)
    lens = [int(x) for x in rng.integers(0, 151, 70)]
    starts = [int(x) for x in rng.integers(0, 200, 70)]
    w, inp, qkv, a, b = packed_case(lens, starts, Hk=1, Hv=2, seed=62)
    c, out, conv, S, _ = run_varlen(G, w, inp, qkv, a, b, lens, starts)
    check_against_singles(G, w, inp, lens, starts, out, conv, S)


def test_varlen_oracle(G):
    """Two sequences against the fp64 oracle, each with its own start."""
    lens, starts = [333, 190], [0, 70]
    w, inp, qkv, a, b = packed_case(lens, starts, seed=63)
    c, out, conv, S, _ = run_varlen(G, w, inp, qkv, a, b, lens, starts)
    cu = cu_of(lens)
    t_out, t_state = tols(w)
    for i, (n, st) in enumerate(zip(lens, starts)):
        ref = oracle_prefill(w, inp, batch_idx=[i], seq_slice=slice(0, n), start_pos=st)
        e_o = rel(out[cu[i]:cu[i + 1]].double().cpu().numpy(), ref["out"][0])
        e_s = rel(S[i].double().cpu().numpy(), ref["S"][0])
        print(f"[varlen oracle seq {i}] out rel {e_o:.3e}, state rel {e_s:.3e}", flush=True)
        assert e_o <= t_out and e_s <= t_state
        assert np.array_equal(I.to_numpy_io(conv[i:i + 1].cpu()), ref["conv_tail"])


def test_varlen_serving_mix(G):
    """Qwen3.6-27B heads (16/48), eight sequences from 1 to 4096 tokens,
    some continuing at a checkpoint position: bitwise equal to single
    calls."""
    lens = [4096, 1, 1000, 3000, 17, 2048, 64, 555]
    starts = [0, 4096, 0, 8192, 100, 0, 64, 4000]
    w, inp, qkv, a, b = packed_case(lens, starts, Hk=16, Hv=48, seed=64)
    c, out, conv, S, _ = run_varlen(G, w, inp, qkv, a, b, lens, starts)
    check_against_singles(G, w, inp, lens, starts, out, conv, S)
