#!/usr/bin/env python3
"""Benchmark of the Gated DeltaNet core on one MI355X.

One step = one chunked-prefill call (front end + chunked rule + final state)
over the Qwen3.6-27B-shaped layer: B=1, L=16384 tokens, 16 key / 48 value
heads, head dims 128, chunk 64, bf16 io, fp32 state, synthetic seeded inputs
resident in HBM, with a workspace allocated once before timing (the call then
runs the two-pass path: chunk-prep kernel + state kernel).  ``value`` is
prefill tokens/s; the fused single-pass kernel is timed beside it.  The same run also times the
one-token decode step of the Qwen3.6-27B-shaped decode workload (B=32, 256
consecutive steps, state ~N(0, 0.05)) and reports its HBM bandwidth, and
times the fp64 CPU oracle on a bounded sample of the prefill workload.
The multi-token decode step (4 tokens per sequence per call) is timed on the
decode workload too, and so is the output gate (RMSNormGated with z): on its
own over the prefill output shape, and fused into the decode step.  The
varlen prefill is timed on a serving-like mix of eight sequences.  Two more
workloads get keys of their own: the Qwen3-Coder-Next-shaped prefill (B=8 x
4096 tokens, 16/32 heads, nonzero initial states) followed by 64 decode steps
from the states it produced, and the 262,144-token Qwen3.6-27B-shaped prefill
that writes 64 checkpoint slots (one per 4096 tokens).  The precise mode
(bf16 hi + lo operands) is timed on the 16k prefill beside the default.

Before every timed region the same call runs untimed for --settle seconds
(default 0.3: the GPU idles while a section generates its inputs on the CPU,
and its clocks take longer than a few calls to come back), then W warm-up
calls, then K timed calls; the JSON line reports the settle as clock_settle.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--settle S] [--only SECTIONS]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GDN prefill tokens/s (MFMA % peak) + decode step HBM GB/s (% peak), 1 GPU"
BF16_PEAK_FLOPS = 2516.6e12      # MI355X dense bf16 MFMA (4096 FLOP/clk/CU x 256 CU x 2.4 GHz)
HBM_PEAK_BYTES = 8.0e12          # MI355X HBM3E


def prefill_flops_per_token_head(C=64, d=128) -> float:
    """Algorithmic FLOPs of the chunked rule per token per value head with the
    triangular products at their exact size: K K^T strictly lower, Q K^T, the
    two T-products and P.Delta lower-inclusive, three C x d x d products
    (W S, Q S, K^T Delta) and the C^3/3 triangular solve."""
    return (C * (C - 1) * d + 4 * C * (C + 1) * d + 6 * C * d * d + C ** 3 / 3) / C


def prefill_bytes(B, L, Hk, Hv, d=128, state_in=False) -> int:
    """Fused-path HBM floor: read qkv, a, b, write o and the final recurrent
    state and conv tail; with state_in, also read the initial ones."""
    conv_dim = 2 * Hk * d + Hv * d
    states = B * (Hv * d * d * 4 + conv_dim * 3 * 2)
    return B * L * (conv_dim * 2 + Hv * 2 * 2 + Hv * d * 2) + (2 if state_in else 1) * states


def varlen_bytes(tokens, B, Hk, Hv, d=128) -> int:
    """HBM floor of a varlen call with initial states: read qkv, a, b, write
    o; read and write every sequence's recurrent state and conv tail."""
    conv_dim = 2 * Hk * d + Hv * d
    return tokens * (conv_dim * 2 + Hv * 2 * 2 + Hv * d * 2) + 2 * B * (Hv * d * d * 4 + conv_dim * 3 * 2)


def decode_bytes(B, Hk, Hv, d=128) -> int:
    """Per decode step: state read + write, qkv, conv state in + out, o, a, b,
    conv taps, A_log and dt_bias."""
    conv_dim = 2 * Hk * d + Hv * d
    return (2 * B * Hv * d * d * 4 + B * conv_dim * 2 + 2 * B * conv_dim * 3 * 2 + B * Hv * d * 2
            + 2 * B * Hv * 2 + conv_dim * 4 * 2 + 2 * Hv * 4)


def profiled_traffic(profile: str, sources):
    """HBM bytes per call from a committed rocprofv3 counter summary
    (FETCH_SIZE + WRITE_SIZE of every kernel the call launches, scaled by a
    copy-kernel calibration), or None when a kernel source changed after the
    counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", profile)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith(("#", "|", "Command")):
            k, _, v = line.partition(":")
            fields[k.strip()] = v.strip()
    csrc = os.path.join(ROOT, "linear_attention_recurrence_causal_amd", "csrc")
    h = hashlib.sha256()
    for f in list(sources) + ["gdn_common.h", "gdn_launch.h"]:
        h.update(open(os.path.join(csrc, f), "rb").read())
    if fields.get("source_sha256") != h.hexdigest() or "traffic_bytes_per_launch" not in fields:
        return None
    return float(fields["traffic_bytes_per_launch"])


PREFILL_SOURCES = ("gdn_prefill_split.hip", "gdn_chunk_common.h")
FUSED_SOURCES = ("gdn_prefill.hip", "gdn_chunk_common.h")
DECODE_SOURCES = ("gdn_decode.hip",)
GATE_SOURCES = ("gdn_gate.hip",)


# seconds of untimed calls before each timed region (set from --settle), and
# the calls that made it for the headline region
SETTLE = {"seconds": 0.0, "headline_calls": None}


def time_events(fn, steps, warmup):
    import torch
    calls = settle_clocks(fn, SETTLE["seconds"])
    if SETTLE["headline_calls"] is None:
        SETTLE["headline_calls"] = calls
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(steps):
        fn()
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / 1e3 / steps   # seconds per call


def settle_clocks(fn, seconds):
    """Untimed calls of fn for `seconds` of wall time, before a timed region's
    warm-up calls: the GPU idles while a section generates its inputs on the
    CPU, and its clocks take longer than a few calls to come back (the 16k
    prefill ran at 0.500 ms per call after 5 untimed calls and at 0.464 ms
    after 200; the Coder-Next prefill at 0.61 ms after 5 and 0.52 ms after
    50).  Returns the calls made."""
    import torch
    n = 0
    if seconds <= 0:
        return n
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end:
        for _ in range(8):
            fn()
        n += 8
        torch.cuda.synchronize()
    return n


def bench_prefill(args):
    """The prefill call as a serving loop makes it for this shape: on a stream
    of its own, with a workspace (allocated once, outside the timed region),
    which selects the two-pass path with the tail of the prep overlapped with
    the state kernel.  Beside it: the same call on the NULL stream (the serial
    two-pass path) and the fused single-pass kernel (no workspace)."""
    import torch
    from linear_attention_recurrence_causal_amd import gdn, inputs as I
    w = I.WORKLOADS[2]
    inp = I.generate(w)
    d = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    cfg = gdn.Config(batch=w.batch, num_k_heads=w.num_k_heads, num_v_heads=w.num_v_heads)
    out = torch.empty(w.batch, w.seq_len, w.num_v_heads, 128, dtype=torch.bfloat16, device="cuda")
    conv = torch.empty(w.batch, w.conv_dim, 3, dtype=torch.bfloat16, device="cuda")
    S = torch.empty(w.batch, w.num_v_heads, 128, 128, device="cuda")
    ws = torch.empty(gdn.prefill_workspace_bytes(cfg, w.seq_len), dtype=torch.uint8, device="cuda")

    def step(workspace):
        gdn.prefill_chunked(cfg, d["qkv"], d["a"], d["b"], d["conv_w"], d["A_log"], d["dt_bias"],
                            None, None, out=out, conv_state_out=conv, rec_state_out=S,
                            workspace=workspace)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        t = time_events(lambda: step(ws), args.steps, args.warmup)
    settle = SETTLE["headline_calls"]
    t_null = time_events(lambda: step(ws), max(2, args.steps // 2), 2)
    t_fused = time_events(lambda: step(None), max(2, args.steps // 4), 1)
    # the precise mode (bf16 hi + lo on the solve's and P Delta's products), both paths
    cfg_p = gdn.Config(batch=w.batch, num_k_heads=w.num_k_heads, num_v_heads=w.num_v_heads,
                       precision=gdn.GDN_PRECISION_HILO)
    ws_p = torch.empty(gdn.prefill_workspace_bytes(cfg_p, w.seq_len), dtype=torch.uint8, device="cuda")

    def step_p(workspace):
        gdn.prefill_chunked(cfg_p, d["qkv"], d["a"], d["b"], d["conv_w"], d["A_log"], d["dt_bias"],
                            None, None, out=out, conv_state_out=conv, rec_state_out=S, workspace=workspace)

    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        t_p = time_events(lambda: step_p(ws_p), max(2, args.steps // 2), 5)
    t_pf = time_events(lambda: step_p(None), 2, 1)
    del ws_p
    tokens = w.batch * w.seq_len
    flops = prefill_flops_per_token_head() * tokens * w.num_v_heads
    byts = prefill_bytes(w.batch, w.seq_len, w.num_k_heads, w.num_v_heads)
    return w, t, t_null, t_fused, (t_p, t_pf), tokens, flops, byts, inp, ws.numel(), settle


def bench_decode(args):
    import torch
    from linear_attention_recurrence_causal_amd import gdn, inputs as I
    w = I.WORKLOADS[1]
    inp = I.generate(w)
    d = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    cfg = gdn.Config(batch=w.batch, num_k_heads=w.num_k_heads, num_v_heads=w.num_v_heads)
    S = d["rec_state"].clone()
    cs = [d["conv_state"].clone(), torch.empty_like(d["conv_state"])]
    out = torch.empty(w.batch, w.num_v_heads, 128, dtype=torch.bfloat16, device="cuda")
    n = w.decode_steps
    state = {"i": 0}

    def step():
        i = state["i"]
        s = i % n
        gdn.decode_step(cfg, d["dec_qkv"][s], d["dec_a"][s], d["dec_b"][s], d["conv_w"],
                        d["A_log"], d["dt_bias"], cs[i % 2], S, out=out,
                        conv_state_out=cs[(i + 1) % 2], rec_state_out=S)
        state["i"] = i + 1

    t = time_events(step, n, args.warmup * 8)
    # The 100.7 MB state fits the 256 MB Infinity Cache (MALL), so consecutive
    # steps may find part of it there.  The same step timed alone after a
    # 512 MiB read that evicts the cache (with clean lines: a write would
    # leave write-backs competing with the step) measures it from HBM.
    flush = torch.ones(1 << 27, device="cuda")
    total = torch.empty((), device="cuda")
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    evs = []
    for k in range(32):
        torch.sum(flush, dim=0, out=total)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        step()
        e1.record(s)
        evs.append((e0, e1))
    torch.cuda.synchronize()
    flushed = sorted(a.elapsed_time(b) / 1e3 for a, b in evs)
    # the ceiling for those bytes from HBM: a plain copy of one state's size
    # (read 100.7 MB, write 100.7 MB), timed the same way after the same read
    src = torch.ones_like(S)
    dst = torch.empty_like(S)
    evs = []
    for k in range(32):
        torch.sum(flush, dim=0, out=total)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        dst.copy_(src)
        e1.record(s)
        evs.append((e0, e1))
    torch.cuda.synchronize()
    copies = sorted(a.elapsed_time(b) / 1e3 for a, b in evs)
    copy_bytes = 2 * S.numel() * 4
    del flush, total, src, dst
    return (w, t, decode_bytes(w.batch, w.num_k_heads, w.num_v_heads), flushed[len(flushed) // 2],
            (copy_bytes, copies[len(copies) // 2]))


def bench_decode_multi(args, T=4):
    """The multi-token step on the same decode workload: T tokens per sequence
    per call (a speculative-decoding verify step), no snapshots."""
    import torch
    from linear_attention_recurrence_causal_amd import gdn, inputs as I
    w = I.WORKLOADS[1]
    d = {k: (None if v is None else v.cuda()) for k, v in I.generate(w).items()}
    cfg = gdn.Config(batch=w.batch, num_k_heads=w.num_k_heads, num_v_heads=w.num_v_heads)
    S = d["rec_state"].clone()
    cs = [d["conv_state"].clone(), torch.empty_like(d["conv_state"])]
    out = torch.empty(w.batch, T, w.num_v_heads, 128, dtype=torch.bfloat16, device="cuda")
    n = w.decode_steps // T
    toks = [tuple(d[k][i * T:(i + 1) * T].transpose(0, 1).contiguous() for k in ("dec_qkv", "dec_a", "dec_b"))
            for i in range(n)]
    state = {"i": 0}

    def call():
        i = state["i"]
        qkv, a, b = toks[i % n]
        gdn.decode_multi(cfg, qkv, a, b, d["conv_w"], d["A_log"], d["dt_bias"], cs[i % 2], S, out=out,
                         conv_state_out=cs[(i + 1) % 2], rec_state_out=S)
        state["i"] = i + 1

    t = time_events(call, n, args.warmup * 4)
    return w, T, t


def bench_output_gate(args):
    """The output gate (RMSNormGated of the core output with z) standalone on
    the prefill output shape [16384, 48, 128] bf16, and fused into the decode
    step of the decode workload (y only, no ungated out)."""
    import torch
    from linear_attention_recurrence_causal_amd import gdn, inputs as I
    w = I.WORKLOADS[2]
    cfg = gdn.Config(batch=w.batch, num_k_heads=w.num_k_heads, num_v_heads=w.num_v_heads)
    gen = torch.Generator().manual_seed(5)
    o = torch.randn((w.seq_len, w.num_v_heads, 128), generator=gen).to(torch.bfloat16).cuda()
    gi = I.gate_inputs(w, (w.seq_len,))
    z, nw = gi["z"].cuda(), gi["norm_w"].cuda()
    y = torch.empty_like(o)
    t = time_events(lambda: gdn.output_gate(cfg, o, z, nw, y=y), args.steps * 4, args.warmup)
    gate_bytes = 3 * o.numel() * 2 + 128 * 2
    del o, z, y

    wd = I.WORKLOADS[1]
    d = {k: (None if v is None else v.cuda()) for k, v in I.generate(wd).items()}
    cfgd = gdn.Config(batch=wd.batch, num_k_heads=wd.num_k_heads, num_v_heads=wd.num_v_heads)
    gd = I.gate_inputs(wd, (wd.decode_steps, wd.batch))
    zd, nwd = gd["z"].cuda(), gd["norm_w"].cuda()
    S = d["rec_state"].clone()
    cs = [d["conv_state"].clone(), torch.empty_like(d["conv_state"])]
    yd = torch.empty(wd.batch, 1, wd.num_v_heads, 128, dtype=torch.bfloat16, device="cuda")
    n = wd.decode_steps
    toks = [tuple(d[k][i:i + 1].transpose(0, 1).contiguous() for k in ("dec_qkv", "dec_a", "dec_b"))
            + (zd[i].unsqueeze(1).contiguous(),) for i in range(n)]
    state = {"i": 0}

    def step():
        i = state["i"]
        qkv, a, b, zz = toks[i % n]
        gdn.decode_gated(cfgd, qkv, a, b, d["conv_w"], d["A_log"], d["dt_bias"], zz, nwd, cs[i % 2], S,
                         y=yd, conv_state_out=cs[(i + 1) % 2], rec_state_out=S)
        state["i"] = i + 1

    td = time_events(step, n, args.warmup * 8)
    dec_bytes = decode_bytes(wd.batch, wd.num_k_heads, wd.num_v_heads) + wd.batch * wd.num_v_heads * 128 * 2
    return {
        "standalone": {"workload": "gdn_output_gate on a [16384, 48, 128] bf16 core output",
                       "us_per_call": t * 1e6,
                       "roofline": {"kernel": "output_gate_kernel", "bound": "hbm",
                                    "achieved": gate_bytes / t / 1e9, "peak": HBM_PEAK_BYTES / 1e9,
                                    "unit": "GB/s", "frac": gate_bytes / t / HBM_PEAK_BYTES,
                                    "traffic": profiled_traffic("output_gate_kernel_qwen36-27b_prefill_16k.md",
                                                                GATE_SOURCES),
                                    "bytes_per_launch": gate_bytes}},
        "fused_decode": {"workload": "gdn_decode_gated, B=32 decode workload, 256 consecutive steps, "
                                    "y only",
                         "us_per_step": td * 1e6, "tokens_per_s": wd.batch / td,
                         "bytes_per_step": dec_bytes,
                         "roofline": {"kernel": "decode_step_kernel (gated, 128 columns per workgroup)",
                                      "bound": "hbm", "achieved": dec_bytes / td / 1e9,
                                      "peak": HBM_PEAK_BYTES / 1e9, "unit": "GB/s",
                                      "frac": dec_bytes / td / HBM_PEAK_BYTES,
                                      "traffic": profiled_traffic("decode_gated_qwen36-27b_decode_b32.md",
                                                                  DECODE_SOURCES)}},
    }


def bench_varlen(args):
    """The varlen prefill on a serving-like mix: eight sequences of 1 to 4096
    tokens (11,381 in all), some continuing from checkpoint positions, with
    the Qwen3.6-27B heads; the same sequences as eight single calls for
    comparison."""
    import torch
    from linear_attention_recurrence_causal_amd import gdn, inputs as I
    lens = [4096, 1, 1000, 3000, 17, 2048, 64, 555]
    starts = [0, 4096, 0, 8192, 100, 0, 64, 4000]
    w = I.Workload("varlen-mix", batch=len(lens), seq_len=max(lens), num_k_heads=16, num_v_heads=48,
                   init_state=True, seed=1005)
    inp = I.generate(w)
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + n)
    qkv = torch.cat([inp["qkv"][i, :n] for i, n in enumerate(lens)]).cuda()
    a = torch.cat([inp["a"][i, :n] for i, n in enumerate(lens)]).cuda()
    b = torch.cat([inp["b"][i, :n] for i, n in enumerate(lens)]).cuda()
    d = {k: inp[k].cuda() for k in ("conv_w", "A_log", "dt_bias", "conv_state", "rec_state")}
    cfg = gdn.Config(batch=w.batch, num_k_heads=16, num_v_heads=48)
    out = torch.empty(cu[-1], 48, 128, dtype=torch.bfloat16, device="cuda")
    conv = torch.empty_like(d["conv_state"])
    S = torch.empty_like(d["rec_state"])
    ws = torch.empty(gdn.prefill_varlen_workspace_bytes(cfg, cu, starts), dtype=torch.uint8, device="cuda")
    t = time_events(lambda: gdn.prefill_varlen(cfg, cu, starts, qkv, a, b, d["conv_w"], d["A_log"], d["dt_bias"],
                                               d["conv_state"], d["rec_state"], out=out, conv_state_out=conv,
                                               rec_state_out=S, workspace=ws), args.steps, args.warmup)
    c1 = gdn.Config(batch=1, num_k_heads=16, num_v_heads=48)
    singles = []
    for i, n in enumerate(lens):
        sl = slice(cu[i], cu[i + 1])
        ws1 = torch.empty(max(gdn.prefill_workspace_bytes(c1, n), 256), dtype=torch.uint8, device="cuda")
        singles.append((qkv[sl].unsqueeze(0), a[sl].unsqueeze(0), b[sl].unsqueeze(0),
                        d["conv_state"][i:i + 1].contiguous(), d["rec_state"][i:i + 1].contiguous(),
                        out[sl].unsqueeze(0), conv[i:i + 1].contiguous(), S[i:i + 1].contiguous(), ws1, starts[i]))

    def all_singles():
        for q, aa, bb, cs, rs, o, co, so, ws1, st in singles:
            gdn.prefill_chunked(c1, q, aa, bb, d["conv_w"], d["A_log"], d["dt_bias"], cs, rs, start_pos=st,
                                out=o, conv_state_out=co, rec_state_out=so, workspace=ws1)

    t1 = time_events(all_singles, max(2, args.steps // 4), 1)
    tokens = cu[-1]
    flops = prefill_flops_per_token_head() * tokens * 48
    return {"workload": f"gdn_prefill_varlen, 8 sequences of {lens} tokens from positions {starts}, 16/48 heads",
            "us_per_call": t * 1e6, "tokens_per_s": tokens / t,
            "roofline": {"kernel": "prep_kernel_varlen + state_kernel<4, VarlenParams>", "bound": "mfma",
                         "achieved": flops / t / 1e12, "peak": BF16_PEAK_FLOPS / 1e12, "unit": "TFLOP/s",
                         "frac": flops / t / BF16_PEAK_FLOPS,
                         "traffic": profiled_traffic("prefill_varlen_serving_mix.md", PREFILL_SOURCES),
                         "hbm_floor_bytes_per_launch": varlen_bytes(tokens, len(lens), 16, 48)},
            "single_calls_us": t1 * 1e6, "speedup_vs_single_calls": t1 / t}


OVERLAPPED = ("two-pass prefill, overlapped: prep_kernel (head chunks), then state_kernel<2> beside "
              "prep_kernel_tail (the other chunks) on disjoint CUs (one call)")


def prefill_roofline(kernel, flops, t, byts, profile):
    return {"kernel": kernel, "bound": "mfma", "achieved": flops / t / 1e12, "peak": BF16_PEAK_FLOPS / 1e12,
            "unit": "TFLOP/s", "frac": flops / t / BF16_PEAK_FLOPS,
            "traffic": profiled_traffic(profile, PREFILL_SOURCES),
            "flops_per_launch": flops, "hbm_floor_bytes_per_launch": byts,
            "hbm_floor_frac": byts / t / HBM_PEAK_BYTES}


def bench_coder(args):
    """Qwen3-Coder-Next-shaped layer: a B=8 x 4096-token chunked prefill (16
    key / 32 value heads, nonzero initial conv and recurrent states, two-pass
    path with a workspace), then 64 one-token decode steps continuing from
    the states that prefill produced."""
    import torch
    from linear_attention_recurrence_causal_amd import gdn, inputs as I
    w = I.WORKLOADS[3]
    d = {k: (None if v is None else v.cuda()) for k, v in I.generate(w).items()}
    cfg = gdn.Config(batch=w.batch, num_k_heads=w.num_k_heads, num_v_heads=w.num_v_heads)
    out = torch.empty(w.batch, w.seq_len, w.num_v_heads, 128, dtype=torch.bfloat16, device="cuda")
    conv = torch.empty_like(d["conv_state"])
    S = torch.empty_like(d["rec_state"])
    ws = torch.empty(gdn.prefill_workspace_bytes(cfg, w.seq_len), dtype=torch.uint8, device="cuda")
    t = time_events(lambda: gdn.prefill_chunked(cfg, d["qkv"], d["a"], d["b"], d["conv_w"], d["A_log"],
                                                d["dt_bias"], d["conv_state"], d["rec_state"], out=out,
                                                conv_state_out=conv, rec_state_out=S, workspace=ws),
                    args.steps, args.warmup)
    del ws
    Sd = S.clone()
    cs = [conv.clone(), torch.empty_like(conv)]
    dout = torch.empty(w.batch, w.num_v_heads, 128, dtype=torch.bfloat16, device="cuda")
    n = w.decode_steps
    state = {"i": 0}

    def dstep():
        i = state["i"]
        k = i % n
        gdn.decode_step(cfg, d["dec_qkv"][k], d["dec_a"][k], d["dec_b"][k], d["conv_w"], d["A_log"],
                        d["dt_bias"], cs[i % 2], Sd, out=dout, conv_state_out=cs[(i + 1) % 2], rec_state_out=Sd)
        state["i"] = i + 1

    # eight sequences move 34.6 MB per step, less than the Python call costs
    # to enqueue: the 64 steps are captured once in a HIP graph and replayed
    for _ in range(2 * n):
        dstep()
    torch.cuda.synchronize()
    state["i"] = 0
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            for _ in range(n):
                dstep()
    torch.cuda.current_stream().wait_stream(side)
    td = time_events(graph.replay, 10, 3) / n
    tokens = w.batch * w.seq_len
    flops = prefill_flops_per_token_head() * tokens * w.num_v_heads
    byts = varlen_bytes(tokens, w.batch, w.num_k_heads, w.num_v_heads)
    bd = decode_bytes(w.batch, w.num_k_heads, w.num_v_heads)
    return {"workload": "Qwen3-Coder-Next-shaped GDN layer: B=8 x 4096-token chunked prefill (16/32 heads, "
                        "nonzero initial states), then 64 decode steps from the produced states",
            "prefill": {"ms_per_call": t * 1e3, "tokens_per_s": tokens / t,
                        "roofline": prefill_roofline("two-pass prefill: prep_kernel + state_kernel<4> (one call)",
                                                     flops, t, byts, "prefill_two_pass_coder_next_b8_4k.md")},
            "decode": {"us_per_step": td * 1e6, "tokens_per_s": w.batch / td, "bytes_per_step": bd,
                       "timing": "64 steps captured in one HIP graph, 10 replays",
                       "roofline": {"kernel": "decode_step_kernel", "bound": "hbm", "achieved": bd / td / 1e9,
                                    "peak": HBM_PEAK_BYTES / 1e9, "unit": "GB/s",
                                    "frac": bd / td / HBM_PEAK_BYTES,
                                    "traffic": profiled_traffic("decode_step_kernel_coder_next_b8.md",
                                                                DECODE_SOURCES)}}}


def bench_long(args):
    """The 262,144-token Qwen3.6-27B-shaped prefill (B=1, 16/48 heads) in one
    call with a workspace, writing a conv + recurrent checkpoint slot every
    4096 tokens (64 slots)."""
    import torch
    from linear_attention_recurrence_causal_amd import gdn, inputs as I
    w = I.WORKLOADS[4]
    d = {k: (None if v is None else v.cuda()) for k, v in I.generate(w).items()}
    cfg = gdn.Config(batch=w.batch, num_k_heads=w.num_k_heads, num_v_heads=w.num_v_heads)
    ents, nb = gdn.state_checkpoint(cfg, 0, w.seq_len, w.ckpt_interval)
    ck = torch.empty(nb, dtype=torch.uint8, device="cuda")
    out = torch.empty(w.batch, w.seq_len, w.num_v_heads, 128, dtype=torch.bfloat16, device="cuda")
    conv = torch.empty(w.batch, w.conv_dim, 3, dtype=torch.bfloat16, device="cuda")
    S = torch.empty(w.batch, w.num_v_heads, 128, 128, device="cuda")
    ws = torch.empty(gdn.prefill_workspace_bytes(cfg, w.seq_len), dtype=torch.uint8, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        t = time_events(lambda: gdn.prefill_chunked(cfg, d["qkv"], d["a"], d["b"], d["conv_w"], d["A_log"],
                                                    d["dt_bias"], None, None, ckpt_interval=w.ckpt_interval,
                                                    ckpt_buf=ck, out=out, conv_state_out=conv, rec_state_out=S,
                                                    workspace=ws),
                        max(2, args.steps // 4), 2)
    tokens = w.batch * w.seq_len
    flops = prefill_flops_per_token_head() * tokens * w.num_v_heads
    byts = prefill_bytes(w.batch, w.seq_len, w.num_k_heads, w.num_v_heads) + len(ents) * (nb // len(ents))
    return {"workload": "Qwen3.6-27B-shaped GDN layer chunked prefill of 262,144 tokens (B=1, 16/48 heads) "
                        "with a checkpoint slot every 4096 tokens (64 slots)",
            "ms_per_call": t * 1e3, "tokens_per_s": tokens / t, "checkpoint_slots": len(ents),
            "roofline": prefill_roofline(OVERLAPPED, flops, t, byts, "prefill_two_pass_qwen36-27b_prefill_256k.md")}


def cpu_baseline(inp, tokens):
    from linear_attention_recurrence_causal_amd import inputs as I
    from oracle import oracle as O
    from tests.helpers import oracle_prefill
    w = I.WORKLOADS[2]
    O.build()
    sl = slice(0, tokens)
    t0 = time.perf_counter()
    oracle_prefill(w, inp, seq_slice=sl)
    dt = time.perf_counter() - t0
    return {"value": tokens * w.batch / dt, "unit": "tokens/s", "cores": O.num_threads(),
            "kind": "oracle",
            "sample": f"fp64 oracle (front end + per-token rule), first {tokens} tokens of the "
                      f"B=1 L={w.seq_len} 16/48-head prefill, all 48 heads, {dt:.1f} s wall"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=50,
                    help="untimed calls before each timed region (the clocks settle within them)")
    ap.add_argument("--settle", type=float, default=0.3,
                    help="seconds of untimed prefill calls before the first warm-up call (the GPU starts idle)")
    ap.add_argument("--cpu-sample-tokens", type=int, default=16384)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--only", default="",
                    help="comma-separated sections to run (prefill, decode, gate, varlen, coder, long, cpu); "
                         "default all.  Without prefill the line has no headline value (for profiling runs)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB fp32 elementwise copy (read 1 GiB, write 1 GiB) "
                         "three times, the reference for scaling HBM byte counters")
    args = ap.parse_args()
    SETTLE["seconds"] = args.settle
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the GDN core shards by (sequence, head) with no "
              "communication, so a multi-GPU figure is N independent copies of this one; "
              "run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)

    sections = {"prefill", "decode", "gate", "varlen", "coder", "long", "cpu"}
    if args.only:
        want = {x.strip() for x in args.only.split(",") if x.strip()}
        bad = want - sections
        if bad:
            ap.error(f"unknown sections {sorted(bad)}")
        sections = want
    if args.no_decode:
        sections -= {"decode", "gate"}
    if args.no_cpu_baseline:
        sections.discard("cpu")
    rec = {"metric": METRIC, "value": None, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": None, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic"}
    inp = None
    if "prefill" in sections:
        print("bench: prefill", file=sys.stderr, flush=True)
        w, t, t_null, t_fused, (t_p, t_pf), tokens, flops, byts, inp, ws_bytes, settled = bench_prefill(args)
        achieved = flops / t
        rec.update({
            "clock_settle": {"seconds": args.settle, "headline_calls": settled,
                             "what": "before every timed region, untimed calls of the same call for this many "
                                     "seconds, then the warm-up calls, so that the timed calls run at the clocks "
                                     "a busy serving loop holds (headline_calls: those of the headline region)"},
            "value": tokens / t,
            "ms_per_step": t * 1e3,
            "config": {"workload": "Qwen3.6-27B-shaped GDN layer chunked prefill", "batch": w.batch,
                       "seq_len": w.seq_len, "num_k_heads": w.num_k_heads,
                       "num_v_heads": w.num_v_heads, "head_dim": 128, "chunk": 64,
                       "io": "bf16", "state": "fp32", "parallelism": "none (1 GPU)"},
            "stream": "a created (non-NULL) stream, as a serving loop runs",
            "roofline": {"kernel": OVERLAPPED,
                         "bound": "mfma", "achieved": achieved / 1e12,
                         "peak": BF16_PEAK_FLOPS / 1e12, "unit": "TFLOP/s",
                         "frac": achieved / BF16_PEAK_FLOPS,
                         "traffic": profiled_traffic("prefill_two_pass_qwen36-27b_prefill_16k.md",
                                                     PREFILL_SOURCES),
                         "flops_per_launch": flops, "hbm_floor_bytes_per_launch": byts,
                         "hbm_floor_frac": byts / t / HBM_PEAK_BYTES,
                         "workspace_bytes": ws_bytes},
            "null_stream": {"what": "the same call on the NULL stream, where the prep runs before the state "
                                    "kernel (serial two-pass path)",
                            "ms_per_call": t_null * 1e3, "tokens_per_s": tokens / t_null,
                            "frac": flops / t_null / BF16_PEAK_FLOPS},
            "fused_path": {"kernel": "prefill_kernel<8>", "ms_per_call": t_fused * 1e3,
                           "tokens_per_s": tokens / t_fused,
                           "frac": flops / t_fused / BF16_PEAK_FLOPS,
                           "traffic": profiled_traffic("prefill_kernel_qwen36-27b_prefill_16k.md",
                                                       FUSED_SOURCES)},
            "precise_mode": {"what": "gdn_config.precision = GDN_PRECISION_HILO (bf16 hi + lo on the "
                                     "triangular solve's and P Delta's products) on the same prefill",
                             "two_pass_ms_per_call": t_p * 1e3, "two_pass_vs_default": t_p / t,
                             "fused_ms_per_call": t_pf * 1e3, "fused_vs_default": t_pf / t_fused},
        })
    if "decode" in sections:
        print("bench: decode", file=sys.stderr, flush=True)
        wd, td, bd, tf, (cb, tc) = bench_decode(args)
        rec["decode"] = {
            "workload": "Qwen3.6-27B-shaped GDN layer decode step, B=32, 256 consecutive steps",
            "us_per_step": td * 1e6, "tokens_per_s": wd.batch / td, "bytes_per_step": bd,
            "roofline": {"kernel": "decode_step_kernel", "bound": "hbm", "achieved": bd / td / 1e9,
                         "peak": HBM_PEAK_BYTES / 1e9, "unit": "GB/s",
                         "frac": bd / td / HBM_PEAK_BYTES,
                         "traffic": profiled_traffic("decode_step_kernel_qwen36-27b_decode_b32.md",
                                                     DECODE_SOURCES)},
            "mall_flushed": {"what": "median of 32 single steps, each after a 512 MiB read that "
                                     "evicts the 256 MB Infinity Cache",
                             "us_per_step": tf * 1e6, "achieved": bd / tf / 1e9, "unit": "GB/s",
                             "frac": bd / tf / HBM_PEAK_BYTES,
                             "cold_copy_ceiling": {"what": "median of 32 plain copies of one state's bytes "
                                                           "(read 100.7 MB, write 100.7 MB), each after "
                                                           "the same 512 MiB read",
                                                   "bytes": cb, "us": tc * 1e6, "achieved": cb / tc / 1e9,
                                                   "frac": cb / tc / HBM_PEAK_BYTES,
                                                   "step_vs_copy_rate": (bd / tf) / (cb / tc)}},
        }
        wm, T, tm = bench_decode_multi(args)
        rec["decode_multi"] = {
            "workload": f"the same decode workload, {T} tokens per sequence per call (verify step)",
            "us_per_call": tm * 1e6, "tokens_per_s": wm.batch * T / tm,
            "speedup_vs_single_steps": T * td / tm}
    if "gate" in sections:
        print("bench: output gate", file=sys.stderr, flush=True)
        rec["output_gate"] = bench_output_gate(args)
    if "varlen" in sections:
        print("bench: varlen prefill", file=sys.stderr, flush=True)
        rec["prefill_varlen"] = bench_varlen(args)
    if "coder" in sections:
        print("bench: coder-next prefill + decode", file=sys.stderr, flush=True)
        rec["coder_next_prefill_decode"] = bench_coder(args)
    if "long" in sections:
        print("bench: 256k prefill with checkpoints", file=sys.stderr, flush=True)
        rec["long_context_256k"] = bench_long(args)
    if "cpu" in sections:
        print("bench: cpu baseline (oracle)", file=sys.stderr, flush=True)
        if inp is None:
            from linear_attention_recurrence_causal_amd import inputs as I
            inp = I.generate(I.WORKLOADS[2])
        rec["cpu_baseline"] = cpu_baseline(inp, args.cpu_sample_tokens)
    if args.calibrate_copy:
        n = 1 << 28
        src = torch.ones(n, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
    rec["gpu"] = torch.cuda.get_device_name(0)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
