"""Seeded synthetic inputs for the Gated DeltaNet core.

This module holds none of the method's arithmetic: it only draws random
tensors of the right shapes and dtypes.  It is the one piece shared by the
fp64 oracle's tests and the HIP path's tests and benchmark.

Shapes follow the pages' two models: the Qwen3.6-27B linear-attention layer
(16 key heads, 48 value heads, head dims 128, conv kernel 4; cortex commit
page "feat(stage-8c): linear-attention layer (Qwen3-Next GatedDeltaNet)",
"Config extended") and the Qwen3-Coder-Next one (16 qk / 32 v heads, head
dim 128; "Add Qwen3-Coder-Next contrib model (80B/3B hybrid DeltaNet+MoE)",
"Model Architecture" table).  Lengths follow the Qwen3.6-27B PR's 16K and
~256K validation runs ("Validation").

Recipe (fixed; every workload uses it):
  * one CPU ``torch.Generator`` seeded with ``seed``; draws in this order: qkv, conv_w, a, b, A_log,
    dt_bias, conv_state, rec_state, then the decode-step qkv, a, b;
  * every draw is fp32 (``torch.randn`` / ``uniform_``), scaled by its
    standard deviation; bf16 tensors are then rounded to bf16 by torch
    (round to nearest even);
  * qkv is drawn in blocks of ``QKV_BLOCK_TOKENS`` tokens (per sequence,
    in order) so that the 256K-token workload never holds an fp32 copy;
  * qkv ~ N(0, 1), conv_w ~ N(0, 0.5), a, b ~ N(0, 1), A_log = ln U(1, 16),
    dt_bias ~ N(0, 0.1), conv_state ~ N(0, 1), rec_state ~ N(0, 0.05)
    (the second parameter of N is the standard deviation).
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np
import torch

QKV_BLOCK_TOKENS = 4096


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seq_len: int            # prefill tokens per sequence (0: decode only)
    num_k_heads: int
    num_v_heads: int
    head_k_dim: int = 128
    head_v_dim: int = 128
    conv_kernel: int = 4
    io: str = "bf16"        # "bf16" or "f32"
    decode_steps: int = 0   # one-token steps after the prefill
    init_state: bool = False  # nonzero initial conv / recurrent state
    ckpt_interval: int = 0
    seed: int = 0
    qkv_std: float = 1.0
    w_std: float = 0.5
    ab_std: float = 1.0
    a_shift: float = 0.0
    b_shift: float = 0.0
    alog_lo: float = 1.0
    alog_hi: float = 16.0
    dt_std: float = 0.1
    conv_std: float = 1.0
    rec_std: float = 0.05
    key_common: float = 0.0  # weight of one shared direction per (sequence, key head) in k

    @property
    def conv_dim(self) -> int:
        return 2 * self.num_k_heads * self.head_k_dim + self.num_v_heads * self.head_v_dim

    @property
    def io_dtype(self) -> torch.dtype:
        return torch.bfloat16 if self.io == "bf16" else torch.float32

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads, by index: the shapes of the pages' models at their lengths.
WORKLOADS = {
    0: Workload("tiny-f32-recurrent", batch=1, seq_len=0, num_k_heads=2, num_v_heads=4,
                head_k_dim=32, head_v_dim=32, io="f32", decode_steps=64, seed=1000),
    1: Workload("qwen3.6-27b-decode-b32", batch=32, seq_len=0, num_k_heads=16, num_v_heads=48,
                decode_steps=256, init_state=True, seed=1001),
    2: Workload("qwen3.6-27b-prefill-16k", batch=1, seq_len=16384, num_k_heads=16,
                num_v_heads=48, seed=1002),
    3: Workload("qwen3-coder-next-prefill-b8-4k+decode64", batch=8, seq_len=4096,
                num_k_heads=16, num_v_heads=32, decode_steps=64, init_state=True, seed=1003),
    4: Workload("qwen3.6-27b-prefill-256k-ckpt4096", batch=1, seq_len=262144, num_k_heads=16,
                num_v_heads=48, ckpt_interval=4096, seed=1004),
}

# Stress variants (same recipe, other distributions).
def slow_decay(w: Workload) -> Workload:
    """A_log = ln U(1e-3, 1e-2): decay per token close to 1, long memory."""
    return w.with_(alog_lo=1e-3, alog_hi=1e-2, name=w.name + "-slowdecay")


def extreme_gates(w: Workload) -> Workload:
    """a, b shifted to about +-30 so softplus / sigmoid sit in their tails."""
    return w.with_(ab_std=1.0, a_shift=30.0, b_shift=-30.0, name=w.name + "-extreme")


def coincident_keys(w: Workload) -> Workload:
    """Keys that nearly coincide (a shared direction of weight 10 against unit
    noise in every k channel, cosine about 0.99 after conv and norm), beta
    near 1 (b shifted by +8) and slow decay: the intra-chunk matrix A then
    has entries near 1 and its powers grow binomially, the hard case of a
    series form of (I + A)^-1."""
    return slow_decay(w).with_(key_common=10.0, b_shift=8.0, name=w.name + "-coincident")


def orthonormal_keys(w: Workload, inp: dict, seed: int = 0) -> dict:
    """Inputs of the store / retrieve / overwrite case (g = 0, beta = 1,
    orthonormal keys): the q and k conv taps become the identity on the
    current token (tap K-1 = 1, the others 0), each token's raw q and k rows
    of a key head are 8 * a basis vector (seeded random index per token, so
    keys repeat and overwrite earlier values, also inside a chunk), a is
    pushed to -30 and b to +30 (softplus and sigmoid in their tails: decay 1,
    beta 1 in fp32), and the initial state is zero.  After the conv, SiLU and
    l2 norm the keys are unit basis vectors.  The v stream keeps its draws."""
    gen = torch.Generator().manual_seed(seed + 31337)
    out = dict(inp)
    B, L, Hk, dk = w.batch, w.seq_len, w.num_k_heads, w.head_k_dim
    kd = Hk * dk
    qkv = inp["qkv"].clone()
    qkv[:, :, : 2 * kd] = 0
    for part in range(2):                      # q, then k
        idx = torch.randint(0, dk, (B, L, Hk), generator=gen)
        rows = torch.zeros(B, L, Hk, dk, dtype=qkv.dtype)
        rows.scatter_(3, idx.unsqueeze(-1), 8.0)
        qkv[:, :, part * kd:(part + 1) * kd] = rows.view(B, L, kd)
    out["qkv"] = qkv
    cw = inp["conv_w"].clone()
    cw[: 2 * kd] = 0
    cw[: 2 * kd, w.conv_kernel - 1] = 1
    out["conv_w"] = cw
    out["a"] = torch.full_like(inp["a"], -30.0)
    out["b"] = torch.full_like(inp["b"], 30.0)
    out["conv_state"] = None if inp["conv_state"] is None else torch.zeros_like(inp["conv_state"])
    out["rec_state"] = None if inp["rec_state"] is None else torch.zeros_like(inp["rec_state"])
    return out


def zero_segments(inp: dict, segments) -> dict:
    """The same inputs with every pre-conv channel of the given token ranges
    [t0, t1) set to zero: the conv output, and with it q, k and v, is zero
    from three tokens into a range until its end, so the l2 norm meets zero
    vectors and the state only decays there."""
    out = dict(inp)
    qkv = inp["qkv"].clone()
    for t0, t1 in segments:
        qkv[:, t0:t1] = 0
    out["qkv"] = qkv
    return out


def _randn(gen, shape, std, dtype):
    x = torch.randn(shape, generator=gen, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)


def generate(w: Workload, seed: int | None = None) -> dict:
    """All inputs of a workload as CPU torch tensors.

    Keys: qkv [B, L, conv_dim], a, b [B, L, H_v] (io dtype); conv_w
    [conv_dim, K] (io); A_log, dt_bias [H_v] fp32; conv_state [B, conv_dim,
    K-1] (io) or None; rec_state [B, H_v, d_k, d_v] fp32 or None;
    dec_qkv [steps, B, conv_dim], dec_a, dec_b [steps, B, H_v] (io) or None.
    """
    seed = w.seed if seed is None else seed
    gen = torch.Generator().manual_seed(seed)
    B, L, Hv, K = w.batch, w.seq_len, w.num_v_heads, w.conv_kernel
    io = w.io_dtype
    qkv = torch.empty((B, L, w.conv_dim), dtype=io)
    for b in range(B):
        for t0 in range(0, L, QKV_BLOCK_TOKENS):
            t1 = min(L, t0 + QKV_BLOCK_TOKENS)
            qkv[b, t0:t1] = _randn(gen, (t1 - t0, w.conv_dim), w.qkv_std, io)
    conv_w = _randn(gen, (w.conv_dim, K), w.w_std, io)
    a = (_randn(gen, (B, L, Hv), w.ab_std, torch.float32) + w.a_shift).to(io)
    b_ = (_randn(gen, (B, L, Hv), w.ab_std, torch.float32) + w.b_shift).to(io)
    A_log = torch.empty(Hv).uniform_(w.alog_lo, w.alog_hi, generator=gen).log_()
    dt_bias = _randn(gen, (Hv,), w.dt_std, torch.float32)
    conv_state = rec_state = None
    if w.init_state:
        conv_state = _randn(gen, (B, w.conv_dim, K - 1), w.conv_std, io)
        rec_state = _randn(gen, (B, Hv, w.head_k_dim, w.head_v_dim), w.rec_std, torch.float32)
    dec_qkv = dec_a = dec_b = None
    if w.decode_steps:
        S = w.decode_steps
        dec_qkv = _randn(gen, (S, B, w.conv_dim), w.qkv_std, io)
        dec_a = (_randn(gen, (S, B, Hv), w.ab_std, torch.float32) + w.a_shift).to(io)
        dec_b = (_randn(gen, (S, B, Hv), w.ab_std, torch.float32) + w.b_shift).to(io)
    if w.key_common:
        # drawn last, so the other inputs match the workload without it
        kd = w.num_k_heads * w.head_k_dim
        base = _randn(gen, (B, 1, kd), w.key_common, torch.float32)
        qkv[:, :, kd:2 * kd] = (qkv[:, :, kd:2 * kd].float() + base).to(io)
    return dict(qkv=qkv, a=a, b=b_, conv_w=conv_w, A_log=A_log, dt_bias=dt_bias,
                conv_state=conv_state, rec_state=rec_state, dec_qkv=dec_qkv, dec_a=dec_a,
                dec_b=dec_b)


def gate_inputs(w: Workload, lead: tuple, seed: int | None = None) -> dict:
    """Inputs of the output gate for core outputs [*lead, H_v, d_v]: z ~ N(0, 1)
    and norm_w ~ N(1, 0.1) (model norm weights start at one), both io dtype.
    Their own generator (seed + 7919), so the layer's inputs are unchanged."""
    seed = (w.seed if seed is None else seed) + 7919
    gen = torch.Generator().manual_seed(seed)
    z = _randn(gen, tuple(lead) + (w.num_v_heads, w.head_v_dim), 1.0, w.io_dtype)
    norm_w = (_randn(gen, (w.head_v_dim,), 0.1, torch.float32) + 1.0).to(w.io_dtype)
    return dict(z=z, norm_w=norm_w)


def to_numpy_io(t: torch.Tensor | None):
    """io tensor -> numpy: bf16 as its uint16 bit pattern, fp32 as float32."""
    if t is None:
        return None
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()
