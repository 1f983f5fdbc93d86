"""Pins of the fp64 oracle against the Python layer the cortex page ported.

The cortex commit page "feat(stage-8c): linear-attention layer (Qwen3-Next
GatedDeltaNet)" says its block was ported from transformers'
``modeling_qwen3_5`` (``Qwen3_5GatedDeltaNet``, ``torch_recurrent_gated_delta_rule``,
``l2norm``, ``Qwen3_5RMSNormGated``; "Block", "Delta rule", "Output").  That
module is importable here, so these CPU tests run it next to the oracle:

  * the whole layer (projections set to channel selections, so the packed
    qkv / a / b / z streams go straight in): pins the [q | k | v] split and
    the key-head offsets of q and k, the conv tap order, SiLU on every conv
    channel, the l2 norm of q and k only, the repeat-interleave head map,
    the discretisation and the gated RMS norm together;
  * its one-token cached-decode conv (``causal_conv1d_update``) on a carried
    conv state: pins the state's column order and that only its last K - 1
    columns matter;
  * its recurrent and chunked rules on given features, with a nonzero
    initial state: pins the rule and the final state;
  * ``Qwen3_5RMSNormGated``: pins the output gate.

The module computes in fp32 and scales q by d_k^-1/2 after its l2 norm;
the oracle runs in fp64 with fp32 io (no bf16 rounding of the conv output)
and ``q_scale = d_k^-1/2``.  A plausible mistake anywhere on these paths (q
and k swapped, a key-head offset off by one head, taps reversed, h % r for
h // r, a missing SiLU, sum for mean in the norm) moves the results by O(1),
far beyond the fp32 tolerance used.
"""
import os

import numpy as np
import pytest
import torch

os.environ.setdefault("HF_HUB_OFFLINE", "1")

hf = pytest.importorskip("transformers.models.qwen3_5.modeling_qwen3_5")
hfc = pytest.importorskip("transformers.models.qwen3_5.configuration_qwen3_5")

from linear_attention_recurrence_causal_amd import inputs as I  # noqa: E402

TOL = 2e-5   # fp32 arithmetic in the ported layer against fp64


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def workload(**kw):
    base = dict(name="hf-pin", batch=2, seq_len=150, num_k_heads=2, num_v_heads=6, head_k_dim=32,
                head_v_dim=32, io="f32", init_state=False, seed=23)
    base.update(kw)
    return I.Workload(**base)


def hf_layer(w, x, norm_w, eps):
    """The ported layer with its projections replaced by channel selections
    of one packed input [qkv | a | b | z], and out_proj selecting the gated
    core output."""
    Hk, Hv, dk, dv = w.num_k_heads, w.num_v_heads, w.head_k_dim, w.head_v_dim
    conv_dim = 2 * Hk * dk + Hv * dv
    hidden = conv_dim + 2 * Hv + Hv * dv
    cfg = hfc.Qwen3_5TextConfig(hidden_size=hidden, linear_num_value_heads=Hv, linear_num_key_heads=Hk,
                                linear_key_head_dim=dk, linear_value_head_dim=dv,
                                linear_conv_kernel_dim=w.conv_kernel, num_hidden_layers=1,
                                layer_types=["linear_attention"], rms_norm_eps=eps, hidden_act="silu")
    layer = hf.Qwen3_5GatedDeltaNet(cfg, 0).float().eval()

    def select(lo, n):
        m = torch.zeros(n, hidden)
        m[torch.arange(n), lo + torch.arange(n)] = 1.0
        return m

    with torch.no_grad():
        layer.in_proj_qkv.weight.copy_(select(0, conv_dim))
        layer.in_proj_a.weight.copy_(select(conv_dim, Hv))
        layer.in_proj_b.weight.copy_(select(conv_dim + Hv, Hv))
        layer.in_proj_z.weight.copy_(select(conv_dim + 2 * Hv, Hv * dv))
        layer.out_proj.weight.copy_(select(0, Hv * dv).t())
        layer.conv1d.weight.copy_(torch.from_numpy(x["conv_w"]).reshape(conv_dim, 1, w.conv_kernel))
        layer.A_log.copy_(torch.from_numpy(x["A_log"]))
        layer.dt_bias.copy_(torch.from_numpy(x["dt_bias"]))
        layer.norm.weight.copy_(torch.from_numpy(norm_w))
        packed = torch.cat([torch.from_numpy(x["qkv"]), torch.from_numpy(x["a"]),
                            torch.from_numpy(x["b"]), torch.from_numpy(x["z"])], dim=-1)
        y = layer(packed)
    return y[..., : Hv * dv].reshape(w.batch, w.seq_len, Hv, dv).double().numpy()


def inputs_of(w):
    g = I.generate(w)
    x = {k: (None if v is None else v.numpy()) for k, v in g.items()}
    gen = torch.Generator().manual_seed(w.seed + 101)
    x["z"] = torch.randn(w.batch, w.seq_len, w.num_v_heads * w.head_v_dim, generator=gen).numpy()
    norm_w = (1.0 + 0.1 * torch.randn(w.head_v_dim, generator=gen)).numpy()
    return x, norm_w


@pytest.mark.parametrize("nk,nv", [(2, 6), (3, 3)])
def test_layer_matches_ported_module(oracle_lib, nk, nv):
    """Front end + rule + gated norm of the oracle == Qwen3_5GatedDeltaNet."""
    from oracle import oracle as O
    w = workload(num_k_heads=nk, num_v_heads=nv)
    x, norm_w = inputs_of(w)
    eps = 1e-6
    want = hf_layer(w, x, norm_w, eps)
    d = O.Dims(w.batch, w.seq_len, w.num_k_heads, w.num_v_heads, w.head_k_dim, w.head_v_dim,
               w.conv_kernel, io_bf16=False, q_scale=w.head_k_dim ** -0.5)
    lay = O.layer(d, x["qkv"], x["a"], x["b"], x["conv_w"], x["A_log"], x["dt_bias"])
    z = x["z"].reshape(w.batch, w.seq_len, w.num_v_heads, w.head_v_dim)
    got = O.output_gate(lay["out"], z, norm_w, eps)
    assert rel(got, want) < TOL
    # every value head on its own (a wrong head map could cancel in a global norm)
    for h in range(w.num_v_heads):
        assert rel(got[:, :, h], want[:, :, h]) < TOL


def test_layer_mistakes_are_caught(oracle_lib):
    """The comparison above is sensitive to the channel split: feeding the
    oracle a stream with the q and k blocks exchanged, or with the key heads
    rotated by one, misses the module by far more than the tolerance."""
    from oracle import oracle as O
    w = workload()
    x, norm_w = inputs_of(w)
    want = hf_layer(w, x, norm_w, 1e-6)
    d = O.Dims(w.batch, w.seq_len, w.num_k_heads, w.num_v_heads, w.head_k_dim, w.head_v_dim,
               w.conv_kernel, io_bf16=False, q_scale=w.head_k_dim ** -0.5)
    Hk, dk = w.num_k_heads, w.head_k_dim
    z = x["z"].reshape(w.batch, w.seq_len, w.num_v_heads, w.head_v_dim)
    kd = Hk * dk
    perms = {
        "q<->k": np.r_[kd:2 * kd, 0:kd, 2 * kd:w.conv_dim],
        "key head +1": np.r_[np.roll(np.arange(kd), dk), kd + np.roll(np.arange(kd), dk),
                             2 * kd:w.conv_dim],
    }
    for name, perm in perms.items():
        lay = O.layer(d, np.ascontiguousarray(x["qkv"][..., perm]), x["a"], x["b"],
                      np.ascontiguousarray(x["conv_w"][perm]), x["A_log"], x["dt_bias"])
        got = O.output_gate(lay["out"], z, norm_w, 1e-6)
        assert rel(got, want) > 1e3 * TOL, name


def test_decode_conv_on_carried_state_matches_ported_update(oracle_lib):
    """The module's cached-decode conv keeps a K-wide state, oldest column
    first, and reads its last K - 1 columns: the oracle's 3-column state
    (oldest -> newest) gives the same conv outputs, token by token."""
    from oracle import oracle as O
    w = workload(seq_len=5, init_state=True)
    x, _ = inputs_of(w)
    d = O.Dims(w.batch, w.seq_len, w.num_k_heads, w.num_v_heads, w.head_k_dim, w.head_v_dim,
               w.conv_kernel, io_bf16=False)
    fe = O.frontend(d, x["qkv"], x["a"], x["b"], x["conv_w"], x["A_log"], x["dt_bias"], x["conv_state"])
    C, K = w.conv_dim, w.conv_kernel
    junk = torch.full((w.batch, C, 1), 1e3)
    state = torch.cat([junk, torch.from_numpy(x["conv_state"])], dim=-1)   # K wide
    weight = torch.from_numpy(x["conv_w"]).reshape(C, K)
    Hk, dk, Hv, dv = w.num_k_heads, w.head_k_dim, w.num_v_heads, w.head_v_dim
    for t in range(w.seq_len):
        xt = torch.from_numpy(x["qkv"][:, t:t + 1]).transpose(1, 2)          # [B, C, 1]
        u = hf.causal_conv1d_update(xt, state, weight, None, "silu")[:, :, 0].double().numpy()
        v_want = u[:, 2 * Hk * dk:].reshape(w.batch, Hv, dv)
        assert rel(fe["v"][:, t], v_want) < 1e-6
        # q, k: the module's l2 norm of the conv output, then compare unit vectors
        qk = torch.from_numpy(u[:, : 2 * Hk * dk]).reshape(w.batch, 2, Hk, dk)
        qn = hf.l2norm(qk[:, 0], dim=-1).numpy()
        kn = hf.l2norm(qk[:, 1], dim=-1).numpy()
        assert rel(fe["q"][:, t], qn) < 1e-6
        assert rel(fe["k"][:, t], kn) < 1e-6
    # the module updated its K-wide state in place: its last K - 1 columns are
    # the oracle's carried state
    tail, _ = O.conv_tail(d, x["qkv"], x["conv_state"])
    assert np.array_equal(state[:, :, 1:].numpy(), tail)


@pytest.mark.parametrize("L", [1, 37, 130])
def test_rule_matches_ported_recurrent_and_chunked(oracle_lib, L):
    """oracle.core on given unit-norm features == the module's recurrent rule
    and its chunked rule (64-token chunks, padded tail), from a nonzero
    initial state; outputs and final state."""
    from oracle import oracle as O
    B, H, dk, dv = 2, 3, 32, 16
    g = torch.Generator().manual_seed(1000 + L)
    q = torch.randn(B, L, H, dk, generator=g)
    k = torch.randn(B, L, H, dk, generator=g)
    v = torch.randn(B, L, H, dv, generator=g)
    gg = -torch.rand(B, L, H, generator=g) * 2.0
    beta = torch.rand(B, L, H, generator=g)
    S0 = 0.05 * torch.randn(B, H, dk, dv, generator=g)
    qs = dk ** -0.5
    qh = np.stack([O.l2_normalize(r, 1e-6, qs) for r in q.double().numpy().reshape(-1, dk)]).reshape(B, L, H, dk)
    kh = np.stack([O.l2_normalize(r, 1e-6, 1.0) for r in k.double().numpy().reshape(-1, dk)]).reshape(B, L, H, dk)
    o_or, S_or = O.core(qh, kh, v.double().numpy(), gg.double().numpy(), beta.double().numpy(),
                        S0.double().numpy())
    for rule in (hf.torch_recurrent_gated_delta_rule, hf.torch_chunk_gated_delta_rule):
        o, S = rule(q, k, v, g=gg, beta=beta, initial_state=S0.clone(), output_final_state=True,
                    use_qk_l2norm_in_kernel=True)
        assert rel(o_or, o.double().numpy()) < TOL, rule.__name__
        assert rel(S_or, S.double().numpy()) < TOL, rule.__name__


def test_output_gate_matches_ported_rmsnormgated(oracle_lib):
    from oracle import oracle as O
    gen = torch.Generator().manual_seed(77)
    for n in (32, 64, 128):
        mod = hf.Qwen3_5RMSNormGated(n, eps=1e-6).float()
        o = torch.randn(40, n, generator=gen) * 3.0
        z = torch.randn(40, n, generator=gen) * 2.0
        with torch.no_grad():
            mod.weight.copy_(1.0 + 0.1 * torch.randn(n, generator=gen))
            want = mod(o, z).double().numpy()
        got = O.output_gate(o.double().numpy(), z.double().numpy(), mod.weight.detach().double().numpy(), 1e-6)
        assert rel(got, want) < 1e-6
