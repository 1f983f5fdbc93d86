"""The entry points enqueue kernels only (no allocation, no synchronisation,
no memset), so a caller can capture them in a HIP graph: decode steps, the
two-pass prefill with its workspace and the output gate are captured with
torch.cuda.graph and replayed several times, with eager work and
synchronisations between the replays, each replay bitwise equal to the same
calls made eagerly on the same inputs.
"""
import pytest
import torch

from linear_attention_recurrence_causal_amd import inputs as I

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def G():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from linear_attention_recurrence_causal_amd import gdn
    return gdn


def test_graph_decode_steps(G):
    """Four decode steps (ping-pong conv states, in-place recurrent state)
    captured once; three replays on new tokens and states."""
    w = I.Workload("graph-decode", batch=4, seq_len=0, num_k_heads=16, num_v_heads=48, decode_steps=16,
                   init_state=True, seed=70)
    d = {k: (None if v is None else v.cuda()) for k, v in I.generate(w).items()}
    c = G.Config(batch=w.batch, num_k_heads=w.num_k_heads, num_v_heads=w.num_v_heads)
    T = 4
    qkv = torch.empty_like(d["dec_qkv"][:T])
    a = torch.empty_like(d["dec_a"][:T])
    b = torch.empty_like(d["dec_b"][:T])
    S = torch.empty_like(d["rec_state"])
    cs = [torch.empty_like(d["conv_state"]), torch.empty_like(d["conv_state"])]
    out = torch.empty(T, w.batch, w.num_v_heads, 128, dtype=torch.bfloat16, device="cuda")

    def steps():
        for t in range(T):
            G.decode_step(c, qkv[t], a[t], b[t], d["conv_w"], d["A_log"], d["dt_bias"], cs[t % 2], S,
                          out=out[t], conv_state_out=cs[(t + 1) % 2], rec_state_out=S)

    def load(r):
        qkv.copy_(d["dec_qkv"][4 * r:4 * r + T])
        a.copy_(d["dec_a"][4 * r:4 * r + T])
        b.copy_(d["dec_b"][4 * r:4 * r + T])
        S.copy_(d["rec_state"] * (1 + r))
        cs[0].copy_(d["conv_state"])

    load(0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        steps()   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        steps()
    for r in range(3):
        load(r)
        steps()
        torch.cuda.synchronize()
        want = (out.clone(), S.clone(), cs[0].clone())
        load(r)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want[0]) and torch.equal(S, want[1]) and torch.equal(cs[0], want[2]), r


def test_graph_prefill_and_gate(G):
    """A two-pass prefill (caller's workspace) followed by the output gate,
    captured once and replayed on three different inputs."""
    w = I.Workload("graph-prefill", batch=2, seq_len=300, num_k_heads=2, num_v_heads=6, init_state=True,
                   seed=71)
    c = G.Config(batch=w.batch, num_k_heads=w.num_k_heads, num_v_heads=w.num_v_heads)
    inputs = [{k: (None if v is None else v.cuda()) for k, v in I.generate(w, seed=71 + r).items()}
              for r in range(3)]
    gates = [{k: v.cuda() for k, v in I.gate_inputs(w, (w.batch, w.seq_len), seed=r).items()} for r in range(3)]
    st = {k: torch.empty_like(v) for k, v in inputs[0].items() if v is not None and k in
          ("qkv", "a", "b", "conv_w", "A_log", "dt_bias", "conv_state", "rec_state")}
    z = torch.empty_like(gates[0]["z"])
    nw = torch.empty_like(gates[0]["norm_w"])
    ws = torch.empty(G.prefill_workspace_bytes(c, w.seq_len), dtype=torch.uint8, device="cuda")
    out = torch.empty(w.batch, w.seq_len, w.num_v_heads, 128, dtype=torch.bfloat16, device="cuda")
    conv = torch.empty_like(st["conv_state"])
    S = torch.empty_like(st["rec_state"])
    y = torch.empty_like(out)

    def call():
        G.prefill_chunked(c, st["qkv"], st["a"], st["b"], st["conv_w"], st["A_log"], st["dt_bias"],
                          st["conv_state"], st["rec_state"], out=out, conv_state_out=conv, rec_state_out=S,
                          workspace=ws)
        G.output_gate(c, out, z, nw, y=y)

    def load(r):
        for k in st:
            st[k].copy_(inputs[r][k])
        z.copy_(gates[r]["z"])
        nw.copy_(gates[r]["norm_w"])

    load(0)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for r in (2, 0, 1):
        load(r)
        call()
        torch.cuda.synchronize()
        want = [t.clone() for t in (out, conv, S, y)]
        for t in (out, conv, S, y):
            t.zero_()
        load(r)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t, u in zip((out, conv, S, y), want):
            assert torch.equal(t, u), r


def test_explicit_stream_argument(G):
    """Calls made with stream= a side stream (outputs and the prefill
    workspace allocated by the binding, recorded on that stream) equal the
    same calls on the current stream bit for bit."""
    w = I.Workload("side-stream", batch=2, seq_len=300, num_k_heads=2, num_v_heads=6, init_state=True,
                   decode_steps=1, seed=72)
    d = {k: (None if v is None else v.cuda()) for k, v in I.generate(w).items()}
    c = G.Config(batch=w.batch, num_k_heads=w.num_k_heads, num_v_heads=w.num_v_heads)
    args = (d["qkv"], d["a"], d["b"], d["conv_w"], d["A_log"], d["dt_bias"], d["conv_state"], d["rec_state"])
    dec = (d["dec_qkv"][0], d["dec_a"][0], d["dec_b"][0], d["conv_w"], d["A_log"], d["dt_bias"],
           d["conv_state"], d["rec_state"])
    want_p = G.prefill_chunked(c, *args)
    want_d = G.decode_step(c, *dec)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    got_p = G.prefill_chunked(c, *args, stream=s)
    got_d = G.decode_step(c, *dec, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for x, y in zip(want_p + want_d, got_p + got_d):
        assert torch.equal(x, y)
