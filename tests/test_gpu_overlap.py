"""The overlapped two-pass prefill: the prep of chunks n1.. runs on a quarter
of the CUs concurrently with the state kernel, which waits for each chunk's
ready flag.  The arithmetic is the serial two-pass path's, so the results
must be bit for bit equal to it (GDN_PREFILL_OVERLAP=0) and within the bars
of the oracle; every tail chunk's flag must end set and the header's error
word zero.  Small shapes force the overlap (GDN_PREFILL_OVERLAP=1); the 16k
workload takes it by default (test_gpu_prefill.py)."""
import contextlib
import math
import os

import pytest
import torch

from linear_attention_recurrence_causal_amd import inputs as I
from tests.helpers import oracle_prefill, to_dev
from tests.test_gpu_prefill import cfg_of, compare, gpu_prefill

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def G():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from linear_attention_recurrence_causal_amd import gdn
    return gdn


@contextlib.contextmanager
def env(**kv):
    old = {k: os.environ.get(k) for k in kv}
    for k, v in kv.items():
        if v is None:
            os.environ.pop(k, None)
        else:
            os.environ[k] = str(v)
    try:
        yield
    finally:
        for k, v in old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


def default_head(c):
    """The library's head fraction: a quarter of the chunks, 30% in the
    precise mode."""
    return 0.30 if c.precision else 0.25


def layout(G, c, w, start_pos, L, head=None):
    """(chunks, n1, byte offset of the flags, 8-byte words per flag row): the
    flags follow the call's records, rows of 32-word multiples, then the
    header."""
    head = default_head(c) if head is None else head
    n = (start_pos + L - 1) // 64 + 1 - start_pos // 64
    per = G.prefill_workspace_bytes(c, 1)            # one chunk: records only
    n1 = min(max(math.ceil(head * n), 1), n - 1)
    return n, n1, n * per, -(-n // 32) * 32


def check_flags(G, c, w, ws, start_pos, L, head):
    """Every tail chunk's flag holds the call's epoch (one nonzero value), no
    error word holds it, and the epoch-tagged counters (40-bit tag, 24-bit
    count) show every state workgroup and every tail item claimed."""
    n, n1, off, frow = layout(G, c, w, start_pos, L, head)
    ng = w.batch * w.num_k_heads
    words = ws[off:off + 8 * (ng * frow + 1024)].view(torch.int64).cpu()
    flags = words[:ng * frow].view(ng, frow)
    hdr = words[ng * frow:]
    tail = flags[:, n1:n]
    epoch = int(tail[0, 0]) & (2 ** 64 - 1)
    assert epoch != 0 and bool((tail == tail[0, 0]).all()), "a tail chunk was never published"
    for word in (512, 544, 576):
        assert int(hdr[word]) & (2 ** 64 - 1) != epoch, f"overlap error word {word}"
    tag = (epoch & (2 ** 40 - 1)) << 24

    def u64(v):
        return int(v) & (2 ** 64 - 1)

    def claims(base):
        return sum(u64(hdr[base + 32 * x]) & 0xffffff for x in range(8)
                   if u64(hdr[base + 32 * x]) & ~0xffffff == tag)
    r = w.num_v_heads // w.num_k_heads
    assert claims(0) == ng * r * 4
    # each persistent tail workgroup claims once more than it processes (the
    # claim that ends its loop): 128 workgroups, 64 in the precise mode
    tail_blocks = 64 if c.precision else 128
    assert claims(256) == ng * (n - n1) + tail_blocks


def run(G, w, d, ws, start_pos=0, seq=slice(None), precision=0, overlap=1, head=None, **kw):
    """One call on a side stream (a created stream: on the NULL stream the
    call takes the serial path)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with env(GDN_PREFILL_OVERLAP=overlap, GDN_PREFILL_OVERLAP_HEAD=head, GDN_PREFILL_STATE_WAVES=2):
        with torch.cuda.stream(side):
            r = gpu_prefill(G, w, d, seq=seq, start_pos=start_pos, workspace=ws, precision=precision, **kw)
    torch.cuda.synchronize()
    return r


CASES = [
    # (name, batch, L, H_k, H_v, start_pos, precision, head fraction)
    ("8/24 L=1000", 1, 1000, 8, 24, 0, 0, None),
    ("B=8 1/2 L=700 from 37", 8, 700, 1, 2, 37, 0, None),
    ("8/16 L=640 precise", 1, 640, 8, 16, 0, 1, None),
    ("8/24 L=1000 head 1 chunk", 1, 1000, 8, 24, 0, 0, 0.01),
    ("8/24 L=1000 head n-1 chunks", 1, 1000, 8, 24, 0, 0, 0.99),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_overlap_bitwise_and_oracle(G, case):
    name, B, L, Hk, Hv, sp, prec, head = case
    w = I.Workload(f"ovl {name}", batch=B, seq_len=sp + L, num_k_heads=Hk, num_v_heads=Hv, init_state=True,
                   seed=91 + B + L)
    inp = I.generate(w)
    d = to_dev(inp)
    precision = G.GDN_PRECISION_HILO if prec else 0
    c = cfg_of(G, w, precision)
    seq = slice(sp, sp + L)
    ws = torch.zeros(G.prefill_workspace_bytes(c, L), dtype=torch.uint8, device="cuda")
    a = run(G, w, d, ws, start_pos=sp, seq=seq, precision=precision, overlap=1, head=head)
    check_flags(G, c, w, ws, sp, L, head)
    b = run(G, w, d, ws, start_pos=sp, seq=seq, precision=precision, overlap=0)
    for x, y in zip(a, b):
        assert torch.equal(x, y), name
    compare(name, w, *a, oracle_prefill(w, inp, seq_slice=seq))


def test_overlap_reused_workspace(G):
    """A second overlapped call on the workspace the first left (its flags all
    set) must wait for its own records: each call's flags carry its own
    epoch, so the first call's flags do not count.
    (Seed 202 is not used for the second input: there head 0's final state is
    token 999's term alone, and one element of that token's v, 31% of its
    norm, lies 8e-6 bf16 ulps from a rounding tie, which the fp32 front end
    and the fp64 oracle round to different neighbours: a 2.3e-3 state
    difference on that head, on every path and in both precision modes.)"""
    B, L, Hk, Hv = 1, 1000, 8, 24
    ws = None
    for i, seed in enumerate((201, 203)):
        w = I.Workload(f"ovl reuse {i}", batch=B, seq_len=L, num_k_heads=Hk, num_v_heads=Hv, init_state=True,
                       seed=seed)
        inp = I.generate(w)
        d = to_dev(inp)
        c = cfg_of(G, w)
        if ws is None:
            ws = torch.zeros(G.prefill_workspace_bytes(c, L), dtype=torch.uint8, device="cuda")
        a = run(G, w, d, ws, overlap=1)
        check_flags(G, c, w, ws, 0, L, None)
        b = run(G, w, d, torch.zeros_like(ws), overlap=0)
        for x, y in zip(a, b):
            assert torch.equal(x, y)
        compare(f"reuse {i}", w, *a, oracle_prefill(w, inp))


def test_overlap_16k_workload(G):
    """The 16k prefill (B=1, 16/48 heads, 256 chunks; the overlap by default)
    on a side stream, bit for bit equal to the serial two-pass path, which
    test_gpu_prefill.py holds to the oracle; flags and counters checked."""
    w = I.WORKLOADS[2]
    inp = I.generate(w)
    d = to_dev(inp)
    c = cfg_of(G, w)
    ws = torch.zeros(G.prefill_workspace_bytes(c, w.seq_len), dtype=torch.uint8, device="cuda")
    a = run(G, w, d, ws, overlap=None, conv_in=None, rec_in=None)
    check_flags(G, c, w, ws, 0, w.seq_len, None)
    b = run(G, w, d, torch.zeros_like(ws), overlap=0, conv_in=None, rec_in=None)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_null_stream_takes_serial_path(G):
    """On the NULL stream the call runs serially: no tail flag is written."""
    w = I.Workload("ovl null", batch=1, seq_len=1000, num_k_heads=8, num_v_heads=24, init_state=True, seed=205)
    inp = I.generate(w)
    d = to_dev(inp)
    c = cfg_of(G, w)
    ws = torch.zeros(G.prefill_workspace_bytes(c, w.seq_len), dtype=torch.uint8, device="cuda")
    with env(GDN_PREFILL_OVERLAP=1, GDN_PREFILL_STATE_WAVES=2):
        a = gpu_prefill(G, w, d, workspace=ws)
    n, n1, off, frow = layout(G, c, w, 0, w.seq_len)
    assert not bool(ws[off:].any())
    b = run(G, w, d, torch.zeros_like(ws), overlap=0)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_overlap_starved_prep_fails_loudly(G):
    """The failure path of the overlap, forced from the host: with the tail
    prep left out (GDN_PREFILL_OVERLAP_SKIP_TAIL=1, so its chunks are never
    published) and a 200 us wait bound, the first wait for a tail chunk runs
    into its bound and every later wait returns at once; the wait error word
    holds the call's epoch and the call's final state and every output row
    come back NaN.  The next call on the same workspace, with its prep, is
    bit for bit the serial one."""
    w = I.Workload("ovl starved", batch=1, seq_len=1000, num_k_heads=8, num_v_heads=24, init_state=True, seed=207)
    inp = I.generate(w)
    d = to_dev(inp)
    c = cfg_of(G, w)
    ws = torch.zeros(G.prefill_workspace_bytes(c, w.seq_len), dtype=torch.uint8, device="cuda")
    with env(GDN_PREFILL_OVERLAP_SKIP_TAIL=1, GDN_PREFILL_OVERLAP_WAIT_US=200):
        out, conv, S = run(G, w, d, ws, overlap=1)
    assert bool(torch.isnan(S).all()), "final state not poisoned"
    assert bool(torch.isnan(out.float()).all()), "output rows not poisoned"
    n, n1, off, frow = layout(G, c, w, 0, w.seq_len)
    ng = w.batch * w.num_k_heads
    hdr = ws[off:off + 8 * (ng * frow + 1024)].view(torch.int64).cpu()[ng * frow:]
    assert int(hdr[576]) != 0, "wait error word not set"
    a = run(G, w, d, ws, overlap=1)
    check_flags(G, c, w, ws, 0, w.seq_len, None)
    b = run(G, w, d, torch.zeros_like(ws), overlap=0)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_overlap_two_streams_in_flight(G):
    """Two overlapped calls on two created streams, enqueued back to back with
    no synchronisation between them (each with its own workspace), share the
    library's two streams: each must come out bit for bit equal to its serial
    run, and each workspace's flags must carry its own call's epoch."""
    w1 = I.Workload("ovl pair a", batch=1, seq_len=1000, num_k_heads=8, num_v_heads=24, init_state=True, seed=211)
    w2 = I.Workload("ovl pair b", batch=1, seq_len=1000, num_k_heads=8, num_v_heads=24, init_state=True, seed=212)
    ins = [I.generate(w) for w in (w1, w2)]
    ds = [to_dev(x) for x in ins]
    cs = [cfg_of(G, w) for w in (w1, w2)]
    wss = [torch.zeros(G.prefill_workspace_bytes(c, w.seq_len), dtype=torch.uint8, device="cuda")
           for c, w in zip(cs, (w1, w2))]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    res = []
    with env(GDN_PREFILL_OVERLAP=1, GDN_PREFILL_STATE_WAVES=2):
        for w, d, ws, s in zip((w1, w2), ds, wss, streams):
            with torch.cuda.stream(s):
                c = cfg_of(G, w)
                res.append(G.prefill_chunked(c, d["qkv"], d["a"], d["b"], d["conv_w"], d["A_log"], d["dt_bias"],
                                             d["conv_state"], d["rec_state"], workspace=ws))
    torch.cuda.synchronize()
    for (w, d, ws, c, r) in zip((w1, w2), ds, wss, cs, res):
        check_flags(G, c, w, ws, 0, w.seq_len, None)
        b = run(G, w, d, torch.zeros_like(ws), overlap=0)
        for x, y in zip(r, b):
            assert torch.equal(x, y), w.name
