"""gdn_prefill_chunked_noalloc: the two-pass prefill on the library's static
scratch array, through the C ABI.  Its results must equal those of
gdn_prefill_chunked with a caller-provided workspace bit for bit (the same
kernels; the static array only changes where the chunk records live and how
many segments a call takes).  Two calls in a row, the second on a smaller
input, so that the second runs on the records the first left behind; then
the precise mode; and the size limit, checked on the host.
"""
import ctypes

import pytest
import torch

from linear_attention_recurrence_causal_amd import inputs as I
from tests.helpers import finite, oracle_prefill, rel, to_dev, tols


@pytest.fixture(scope="module")
def G():
    from linear_attention_recurrence_causal_amd import gdn
    return gdn


def cfg_of(G, w, precision=0):
    return G.Config(batch=w.batch, num_k_heads=w.num_k_heads, num_v_heads=w.num_v_heads, precision=precision)


def both(G, w, start_pos=0, ckpt_interval=0, precision=0):
    """The workload through the static-scratch entry and through
    gdn_prefill_chunked with a whole-call workspace; returns both results
    (out, conv, state, checkpoint buffer)."""
    d = to_dev(I.generate(w))
    c = cfg_of(G, w, precision)
    res = []
    for noalloc in (True, False):
        ck = None
        if ckpt_interval:
            _, nb = G.state_checkpoint(c, start_pos, w.seq_len, ckpt_interval)
            ck = torch.zeros(nb, dtype=torch.uint8, device="cuda")
        args = (c, d["qkv"], d["a"], d["b"], d["conv_w"], d["A_log"], d["dt_bias"], d["conv_state"],
                d["rec_state"])
        kw = dict(start_pos=start_pos, ckpt_interval=ckpt_interval, ckpt_buf=ck)
        if noalloc:
            r = G.prefill_chunked_noalloc(*args, **kw)
        else:
            r = G.prefill_chunked(*args, workspace="auto", **kw)
        torch.cuda.synchronize()
        res.append(tuple(r) + (ck,))
    return res


def assert_equal(tag, a, b):
    for name, x, y in zip(("out", "conv", "state", "ckpt"), a, b):
        if x is None:
            assert y is None
            continue
        assert torch.equal(x, y), f"{tag}: {name} differs"
    print(f"[{tag}] equal to the workspace call bit for bit", flush=True)


@pytest.mark.gpu
def test_noalloc_equals_workspace_call_twice(G):
    """First call: 4 sequences of 4096 tokens, Qwen3.6-27B heads (16/48),
    initial states, checkpoints every 1024 tokens; its records (4.6 MiB per
    chunk) take 5 segments of the 64 MiB array.  Second call, smaller: one
    sequence of 300 tokens from position 37 with 2/4 heads, on the array the
    first call left.  Both bit for bit equal to gdn_prefill_chunked with a
    whole-call workspace; the second also against the oracle."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    w1 = I.Workload("noalloc-1", batch=4, seq_len=4096, num_k_heads=16, num_v_heads=48, init_state=True,
                    seed=71)
    per_chunk = G.prefill_workspace_bytes(cfg_of(G, w1), 1)
    assert 4 <= G.NOALLOC_SCRATCH_BYTES // per_chunk < 4096 // 64   # several segments
    a, b = both(G, w1, ckpt_interval=1024)
    assert_equal("noalloc B=4 L=4096 16/48", a, b)
    assert finite(a[0], a[2])

    w2 = I.Workload("noalloc-2", batch=1, seq_len=300, num_k_heads=2, num_v_heads=4, init_state=True, seed=72)
    a, b = both(G, w2, start_pos=37)
    assert_equal("noalloc B=1 L=300 2/4 from 37", a, b)
    inp = I.generate(w2)
    ref = oracle_prefill(w2, inp, start_pos=37)
    t_out, t_state = tols(w2)
    e_out, e_state = rel(a[0].double().cpu().numpy(), ref["out"]), rel(a[2].double().cpu().numpy(), ref["S"])
    print(f"[noalloc small] out rel {e_out:.3e}, state rel {e_state:.3e}", flush=True)
    assert e_out <= t_out and e_state <= t_state


@pytest.mark.gpu
def test_noalloc_precise_mode(G):
    """The precise mode's larger records (26624 bytes per value head and
    chunk) on the static array, two segments: equal to the workspace call."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    w = I.Workload("noalloc-3", batch=2, seq_len=2000, num_k_heads=16, num_v_heads=48, init_state=True,
                   seed=73)
    a, b = both(G, w, precision=G.GDN_PRECISION_HILO)
    assert_equal("noalloc precise B=2 L=2000 16/48", a, b)


def test_noalloc_rejects_records_beyond_the_array(G):
    """Host check, before any device call: one chunk's records above the
    64 MiB array give GDN_ESPACE; a bad config gives GDN_EINVAL."""
    P = ctypes.c_void_p
    fake = 1 << 34

    def call(c):
        return G.lib.gdn_prefill_chunked_noalloc(ctypes.byref(c.c()), 64, 0, P(fake), P(fake * 2), P(fake * 3),
                                                 P(fake * 4), P(fake * 5), P(fake * 6), None, P(fake * 7),
                                                 None, P(fake * 8), P(fake * 9), None, 0, 0, None)
    # B = 58 sequences of 16/48 heads: one chunk is 58 * (16 * 32768 + 48 * 13568) bytes > 64 MiB
    big = G.Config(batch=58, num_k_heads=16, num_v_heads=48)
    assert G.prefill_workspace_bytes(big, 1) > G.NOALLOC_SCRATCH_BYTES
    assert call(big) == G.GDN_ESPACE
    fits = G.Config(batch=57, num_k_heads=16, num_v_heads=48)
    assert G.prefill_workspace_bytes(fits, 1) <= G.NOALLOC_SCRATCH_BYTES
    # precise records: 38 * (16 * 32768 + 48 * 26624) bytes > 64 MiB
    precise = G.Config(batch=38, num_k_heads=16, num_v_heads=48, precision=G.GDN_PRECISION_HILO)
    assert G.prefill_workspace_bytes(precise, 1) > G.NOALLOC_SCRATCH_BYTES
    assert call(precise) == G.GDN_ESPACE
    assert call(G.Config(batch=1, num_k_heads=16, num_v_heads=47)) == G.GDN_EINVAL
