"""Shared helpers of the test-suite: oracle runs and comparisons.

The oracle side only ever sees inputs from the seeded generators; nothing
the HIP path produces is fed to it.
"""
from __future__ import annotations

import numpy as np
import torch

from linear_attention_recurrence_causal_amd import inputs as I

# Bars (relative L2 over the whole compared tensor).
TOL_F32 = 1e-4          # fp32-io workloads: outputs and state
TOL_BF16_OUT = 1e-2     # bf16-io workloads: outputs
TOL_BF16_STATE = 2e-3   # bf16-io workloads: recurrent state (fp32)


def rel(x, ref) -> float:
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / (den if den > 0 else 1.0))


def tols(w: I.Workload):
    return (TOL_F32, TOL_F32) if w.io == "f32" else (TOL_BF16_OUT, TOL_BF16_STATE)


def dims(w: I.Workload, seq_len=None, batch=None, **kw):
    from oracle.oracle import Dims
    return Dims(w.batch if batch is None else batch, w.seq_len if seq_len is None else seq_len,
                w.num_k_heads, w.num_v_heads, w.head_k_dim, w.head_v_dim, w.conv_kernel,
                io_bf16=(w.io == "bf16"), **kw)


def np_io(t):
    return I.to_numpy_io(t)


def io_to_f64(x):
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def round_like_io(x64, w: I.Workload):
    """What the GPU stores for an fp64 oracle output: RNE to the io dtype."""
    t = torch.from_numpy(np.ascontiguousarray(x64))
    return t.to(w.io_dtype).double().numpy()


def oracle_prefill(w: I.Workload, inp: dict, batch_idx=None, heads=None, start_pos=0,
                   seq_slice=None, conv_state=None, S0=None, want_ckpt=False, ckpt_interval=0):
    """Oracle over (a slice of) the prefill tokens for selected sequences / heads.

    conv_state / S0 override the workload's initial state (S0 in fp64)."""
    from oracle import oracle as O
    sl = slice(None) if seq_slice is None else seq_slice
    bi = list(range(w.batch)) if batch_idx is None else list(batch_idx)
    qkv = np_io(inp["qkv"][bi][:, sl])
    a = np_io(inp["a"][bi][:, sl])
    b = np_io(inp["b"][bi][:, sl])
    if conv_state is None and inp["conv_state"] is not None:
        conv_state = np_io(inp["conv_state"][bi])
    if S0 is None and inp["rec_state"] is not None:
        S0 = inp["rec_state"][bi].double().numpy()
    d = dims(w, seq_len=qkv.shape[1], batch=len(bi), start_pos=start_pos,
             ckpt_interval=ckpt_interval)
    res = O.layer(d, qkv, a, b, np_io(inp["conv_w"]), inp["A_log"].numpy(),
                  inp["dt_bias"].numpy(), conv_state, S0, heads=heads, want_ckpt=want_ckpt)
    tail, ck = O.conv_tail(d, qkv, conv_state, want_ckpt=want_ckpt)
    res["conv_tail"] = tail
    res["ckpt_conv"] = ck
    return res


def oracle_decode(w: I.Workload, inp: dict, steps: int, batch_idx=None, heads=None,
                  conv_state=None, S0=None):
    """Oracle of `steps` one-token steps == the rule over those tokens as one
    sequence (the oracle's split-anywhere continuation is bitwise)."""
    from oracle import oracle as O
    bi = list(range(w.batch)) if batch_idx is None else list(batch_idx)
    qkv = np_io(inp["dec_qkv"][:steps, bi].transpose(0, 1).contiguous())
    a = np_io(inp["dec_a"][:steps, bi].transpose(0, 1).contiguous())
    b = np_io(inp["dec_b"][:steps, bi].transpose(0, 1).contiguous())
    if conv_state is None and inp["conv_state"] is not None:
        conv_state = np_io(inp["conv_state"][bi])
    if S0 is None and inp["rec_state"] is not None:
        S0 = inp["rec_state"][bi].double().numpy()
    d = dims(w, seq_len=steps, batch=len(bi))
    res = O.layer(d, qkv, a, b, np_io(inp["conv_w"]), inp["A_log"].numpy(),
                  inp["dt_bias"].numpy(), conv_state, S0, heads=heads)
    tail, _ = O.conv_tail(d, qkv, conv_state)
    res["conv_tail"] = tail
    return res


def to_dev(inp: dict, device="cuda"):
    return {k: (None if v is None else v.to(device)) for k, v in inp.items()}


def finite(*ts) -> bool:
    return all(bool(torch.isfinite(t.float()).all()) for t in ts)
