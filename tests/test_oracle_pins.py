"""Pins of the fp64 oracle against facts fixed by the pages and by mathematics.

Nothing here compares the oracle with a retyped copy of itself: each test
uses a closed form, a hand-computed example, an invariant, a library routine
for a textbook special case, brute force with explicit matrices, or the
structurally different chunked formulation.  The pages this follows:
  * cortex commit "feat(stage-8c): linear-attention layer (Qwen3-Next
    GatedDeltaNet)": "Block", "Discretisation", "Delta rule", "State",
    "8 unit tests" (softplus branches, l2norm hand case and zero vector,
    repeat-interleave round trip, no NaN/Inf);
  * "Add Qwen3.6-27B hybrid DeltaNet/GQA contrib model and vLLM serving
    path": "Summary" (recurrent and conv checkpoints for prefix reuse).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import chunked_ref
from linear_attention_recurrence_causal_amd import inputs as I

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def dims_of(w, **kw):
    from oracle.oracle import Dims
    return Dims(w.batch, w.seq_len, w.num_k_heads, w.num_v_heads, w.head_k_dim, w.head_v_dim,
                w.conv_kernel, io_bf16=(w.io == "bf16"), **kw)


def np_inputs(w, seed=None):
    """The workload's inputs as numpy: io tensors as bf16 bits / fp32, the
    initial recurrent state as fp64."""
    n = {}
    for k, v in I.generate(w, seed).items():
        if v is None:
            n[k] = None
        elif k in ("A_log", "dt_bias"):
            n[k] = v.numpy()
        elif k == "rec_state":
            n[k] = v.double().numpy()
        else:
            n[k] = I.to_numpy_io(v)
    return n


def io_to_f64(x):
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


# ---------------------------------------------------------------- scalars

def test_bf16_rounding_matches_torch_on_fp32_values(oracle_lib):
    """RNE to bf16 is a library routine in torch (fp32 -> bf16); on inputs
    that are fp32 values the fp64 rounding must agree bit for bit."""
    g = torch.Generator().manual_seed(7)
    x = torch.cat([torch.randn(4000, generator=g) * s for s in (1e-30, 1e-3, 1.0, 1e3, 1e30)])
    # exact ties (odd multiple of half a bf16 ulp) in both directions
    ties = torch.tensor([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 2 ** -126 * (1 + 2 ** -8)])
    x = torch.cat([x, ties])
    want = x.to(torch.bfloat16).double().numpy()
    got = np.array([oracle_lib.round_bf16(float(v)) for v in x.double().numpy()])
    assert np.array_equal(got, want)
    assert oracle_lib.round_bf16(1 + 2 ** -8) == 1.0           # tie -> even
    assert oracle_lib.round_bf16(1 + 3 * 2 ** -8) == 1 + 2 ** -6  # tie -> even (up)
    assert oracle_lib.round_bf16(0.0) == 0.0


def test_softplus_branches(oracle_lib):
    """The small/large branches the cortex tests name: exact values."""
    assert oracle_lib.softplus(0.0) == pytest.approx(math.log(2.0), rel=1e-15)
    # log(1 + e^-30) = e^-30 - e^-60/2 + ...  (e^-30 = 9.357622968840175e-14)
    assert oracle_lib.softplus(-30.0) == pytest.approx(9.357622968839737e-14, rel=1e-13)
    assert oracle_lib.softplus(30.0) - 30.0 == pytest.approx(9.357622968839737e-14, rel=1e-2)
    # sp(x) - sp(-x) = x and sp(x) >= max(x, 0) for all x
    for x in np.linspace(-40, 40, 161):
        assert oracle_lib.softplus(x) - oracle_lib.softplus(-x) == pytest.approx(x, abs=1e-12)
        assert oracle_lib.softplus(x) >= max(x, 0.0)
    # large branch: within 2.1e-9 of x beyond 20 (fp32 cannot see the difference)
    assert abs(oracle_lib.softplus(20.0) - 20.0) < 2.1e-9
    # a naive fp32 log(1 + exp(x)) gives exactly 0 at -30; the oracle must not
    assert float(np.log(np.float32(1) + np.exp(np.float32(-30.0)))) == 0.0
    assert oracle_lib.softplus(-30.0) > 0


def test_sigmoid_silu_closed_forms(oracle_lib):
    assert oracle_lib.sigmoid(0.0) == 0.5
    for x in (-35.0, -3.0, -0.25, 0.7, 5.0, 35.0):
        assert oracle_lib.sigmoid(x) + oracle_lib.sigmoid(-x) == pytest.approx(1.0, abs=1e-15)
        want = float(torch.nn.functional.silu(torch.tensor(x, dtype=torch.float64)))
        assert oracle_lib.silu(x) == pytest.approx(want, rel=1e-14, abs=1e-300)
    assert oracle_lib.silu(0.0) == 0.0


def test_discretisation_closed_form(oracle_lib):
    """A_log = 0, a + dt_bias = 0: g = -softplus(0) = -ln 2, so exp(g) = 1/2."""
    g = oracle_lib.gate_g(0.0, 0.25, -0.25)
    assert g == pytest.approx(-math.log(2.0), rel=1e-15)
    assert math.exp(g) == pytest.approx(0.5, rel=1e-15)
    # A_log = ln 3 scales the softplus by 3; large negative input: g -> 0-
    assert oracle_lib.gate_g(math.log(3.0), 1.0, 0.0) == pytest.approx(-3 * math.log1p(math.e),
                                                                      rel=1e-14)
    assert -1e-12 < oracle_lib.gate_g(0.0, -30.0, 0.0) < 0.0


def test_l2norm_hand_case_and_zero(oracle_lib):
    """(3, 4) -> (3, 4) / sqrt(25 + 1e-6); 0 -> 0 (finite)."""
    y = oracle_lib.l2_normalize([3.0, 4.0], eps=1e-6)
    s = 1.0 / 5.0 * (1.0 - 2e-8 + 1.5 * (4e-8) ** 2 / 4)  # (25(1+4e-8))^(-1/2) by series
    assert y[0] == pytest.approx(3 * s, rel=1e-15)
    assert y[1] == pytest.approx(4 * s, rel=1e-15)
    assert y[0] == pytest.approx(0.599999988, rel=1e-9)
    z = oracle_lib.l2_normalize(np.zeros(128), eps=1e-6)
    assert np.all(z == 0.0) and np.all(np.isfinite(z))
    # scale folds in multiplicatively
    y2 = oracle_lib.l2_normalize([3.0, 4.0], eps=1e-6, scale=0.5)
    assert np.allclose(y2, 0.5 * y, rtol=1e-15)


# ---------------------------------------------------------------- output gate

def test_output_gate_hand_case(oracle_lib):
    """[GDN] "Output", RMSNormGated: o = (3, 4), eps = 0, w = 1: mean(o^2) =
    25/2, so o / rms = (3, 4) sqrt(2) / 5; with z = 50 (silu(50) = 50 (1 -
    e^-50 + ...)) y = (30 sqrt 2, 40 sqrt 2) to 1e-15."""
    y = oracle_lib.output_gate([[3.0, 4.0]], [[50.0, 50.0]], [1.0, 1.0], eps=0.0)
    assert y[0, 0] == pytest.approx(30 * math.sqrt(2.0), rel=1e-15)
    assert y[0, 1] == pytest.approx(40 * math.sqrt(2.0), rel=1e-15)
    # z = 0 closes the gate, w scales each channel on its own
    assert np.all(oracle_lib.output_gate([[3.0, 4.0]], [[0.0, 0.0]], [1.0, 1.0]) == 0.0)
    y2 = oracle_lib.output_gate([[3.0, 4.0]], [[50.0, 50.0]], [2.0, -0.5], eps=0.0)
    assert y2[0, 0] == pytest.approx(60 * math.sqrt(2.0), rel=1e-15)
    assert y2[0, 1] == pytest.approx(-20 * math.sqrt(2.0), rel=1e-15)


def test_output_gate_mean_not_sum_and_scale_invariance(oracle_lib):
    """A constant row c (n channels, eps = 0) normalises to sign(c) for every
    n, which holds for the mean of squares only; o -> a o with eps -> a^2
    eps leaves y unchanged."""
    for n in (2, 32, 128):
        for c in (0.01, -3.0, 700.0):
            y = oracle_lib.output_gate(np.full((1, n), c), np.full((1, n), 60.0), np.ones(n), eps=0.0)
            assert np.allclose(y, math.copysign(60.0, c), rtol=1e-14)
    rng = np.random.default_rng(5)
    o, z, w = rng.standard_normal((6, 128)), rng.standard_normal((6, 128)), rng.standard_normal(128)
    for a in (1e-3, 7.0):
        assert rel(oracle_lib.output_gate(a * o, z, w, eps=1e-6 * a * a),
                   oracle_lib.output_gate(o, z, w, eps=1e-6)) < 1e-14


def test_output_gate_matches_torch_rms_norm(oracle_lib):
    """The textbook RMSNorm of torch (fp64, weight w, the same eps) times
    torch's SiLU of z, on random rows of 32, 64 and 128 channels."""
    rng = np.random.default_rng(6)
    for n in (32, 64, 128):
        o = rng.standard_normal((40, n)) * rng.uniform(0.01, 10.0, (40, 1))
        z, w = 3 * rng.standard_normal((40, n)), rng.standard_normal(n)
        to = lambda x: torch.from_numpy(np.ascontiguousarray(x))
        want = (torch.nn.functional.rms_norm(to(o), (n,), to(w), eps=1e-6)
                * torch.nn.functional.silu(to(z))).numpy()
        assert rel(oracle_lib.output_gate(o, z, w, eps=1e-6), want) < 1e-14


# ---------------------------------------------------------------- front end

def small_workload(**kw):
    base = dict(name="pin", batch=2, seq_len=11, num_k_heads=2, num_v_heads=4, head_k_dim=8,
                head_v_dim=8, io="bf16", init_state=True, seed=11)
    base.update(kw)
    return I.Workload(**base)


def test_conv_matches_library_correlation(oracle_lib):
    """Causal depthwise conv == numpy cross-correlation over the state-prepended
    stream (tap K-1 weights the current token); SiLU from torch; bf16 RNE."""
    from oracle import oracle as O
    w = small_workload()
    x = np_inputs(w)
    dims = dims_of(w)
    fe = O.frontend(dims, x["qkv"], x["a"], x["b"], x["conv_w"], x["A_log"], x["dt_bias"],
                    x["conv_state"])
    qkv = io_to_f64(x["qkv"])
    cs = io_to_f64(x["conv_state"])
    cw = io_to_f64(x["conv_w"])
    Hk, dk, dv = w.num_k_heads, w.head_k_dim, w.head_v_dim
    for b in range(w.batch):
        for h in range(w.num_v_heads):
            for j in range(dv):
                c = 2 * Hk * dk + h * dv + j
                stream = np.concatenate([cs[b, c], qkv[b, :, c]])
                y = np.correlate(stream, cw[c], mode="valid")
                u = torch.nn.functional.silu(torch.from_numpy(y)).float().to(torch.bfloat16)
                assert np.array_equal(fe["v"][b, :, h, j], u.double().numpy())


def test_conv_one_hot_taps_and_zero_state(oracle_lib):
    """w = e_{K-1}: u_t = SiLU(x_t); w = e_0: u_t = SiLU(x_{t-3}), reading the
    carried state for t < 3; a missing state acts as zero padding."""
    from oracle import oracle as O
    w = small_workload(io="f32")
    x = np_inputs(w)
    dims = dims_of(w, round_conv=False)
    C, K = w.conv_dim, w.conv_kernel
    silu = lambda t: torch.nn.functional.silu(torch.from_numpy(t)).numpy()
    for tap in (K - 1, 0):
        cw = np.zeros((C, K), np.float32)
        cw[:, tap] = 1.0
        fe = O.frontend(dims, x["qkv"], x["a"], x["b"], cw, x["A_log"], x["dt_bias"],
                        x["conv_state"])
        voff = 2 * w.num_k_heads * w.head_k_dim
        v_ch = x["qkv"][:, :, voff:].astype(np.float64).reshape(w.batch, w.seq_len,
                                                               w.num_v_heads, w.head_v_dim)
        if tap == K - 1:
            assert np.allclose(fe["v"], silu(v_ch), rtol=1e-14, atol=0)
        else:
            st = x["conv_state"][:, voff:, 0].astype(np.float64)  # oldest state column
            want = np.concatenate(
                [np.broadcast_to(st.reshape(w.batch, 1, w.num_v_heads, w.head_v_dim),
                                 (w.batch, 1, w.num_v_heads, w.head_v_dim)),
                 x["conv_state"][:, voff:, 1:].astype(np.float64).transpose(0, 2, 1).reshape(
                     w.batch, K - 2, w.num_v_heads, w.head_v_dim),
                 v_ch[:, : w.seq_len - (K - 1)]], axis=1)
            assert np.allclose(fe["v"], silu(want), rtol=1e-14, atol=0)
    # zero conv state == no conv state
    zero = np.zeros_like(x["conv_state"])
    a = O.frontend(dims, x["qkv"], x["a"], x["b"], x["conv_w"], x["A_log"], x["dt_bias"], zero)
    b = O.frontend(dims, x["qkv"], x["a"], x["b"], x["conv_w"], x["A_log"], x["dt_bias"], None)
    for k in a:
        assert np.array_equal(a[k], b[k])


def test_conv_tail_is_a_bit_copy(oracle_lib):
    """Carried conv state = the last K-1 pre-conv inputs, bit for bit; for a
    call shorter than K-1 tokens part of it still comes from the old state."""
    from oracle import oracle as O
    for L in (11, 2, 0):
        w = small_workload(seq_len=L)
        x = np_inputs(w)
        tail, _ = O.conv_tail(dims_of(w), x["qkv"], x["conv_state"])
        ext = np.concatenate([x["conv_state"], x["qkv"].transpose(0, 2, 1)], axis=2)
        assert np.array_equal(tail, ext[:, :, L:L + 3])


def test_qk_unit_norm_and_gates(oracle_lib):
    from oracle import oracle as O
    w = small_workload()
    x = np_inputs(w)
    fe = O.frontend(dims_of(w), x["qkv"], x["a"], x["b"], x["conv_w"], x["A_log"],
                    x["dt_bias"], x["conv_state"])
    nq = np.linalg.norm(fe["q"], axis=-1)
    nk = np.linalg.norm(fe["k"], axis=-1)
    assert np.all(nq < 1.0) and np.all(nq > 1.0 - 1e-3)
    assert np.all(nk < 1.0) and np.all(nk > 1.0 - 1e-3)
    a = io_to_f64(x["a"])
    b = io_to_f64(x["b"])
    # softplus / sigmoid from torch (library routines)
    sp = torch.nn.functional.softplus(torch.from_numpy(a + x["dt_bias"].astype(np.float64)),
                                      threshold=1000).numpy()
    g_want = -np.exp(x["A_log"].astype(np.float64)) * sp
    assert np.allclose(fe["g"], g_want, rtol=1e-13)
    assert np.allclose(fe["beta"], torch.sigmoid(torch.from_numpy(b)).numpy(), rtol=1e-14)
    assert np.all(fe["g"] < 0) and np.all((fe["beta"] > 0) & (fe["beta"] < 1))


def test_repeat_interleave_head_map(oracle_lib):
    """Value head h reads key head h // (H_v/H_k): the layer equals the
    chunked reference run on numpy.repeat(q, r) (interleaved copies), and
    repeating then regrouping is the identity (the cortex round-trip test)."""
    from oracle import oracle as O
    w = small_workload(num_k_heads=2, num_v_heads=6, seq_len=9)
    x = np_inputs(w)
    dims = dims_of(w)
    fe = O.frontend(dims, x["qkv"], x["a"], x["b"], x["conv_w"], x["A_log"], x["dt_bias"],
                    x["conv_state"])
    r = w.num_v_heads // w.num_k_heads
    qr = np.repeat(fe["q"], r, axis=2)
    kr = np.repeat(fe["k"], r, axis=2)
    assert np.array_equal(qr.reshape(*qr.shape[:2], w.num_k_heads, r, -1)[:, :, :, 0], fe["q"])
    lay = O.layer(dims, x["qkv"], x["a"], x["b"], x["conv_w"], x["A_log"], x["dt_bias"],
                  x["conv_state"], x["rec_state"])
    for b in range(w.batch):
        for h in range(w.num_v_heads):
            o, S = chunked_ref.chunked_head(qr[b, :, h], kr[b, :, h], fe["v"][b, :, h],
                                            fe["g"][b, :, h], fe["beta"][b, :, h],
                                            x["rec_state"][b, h], chunk=4)
            assert rel(lay["out"][b, :, h], o) < 1e-12
            assert rel(lay["S"][b, h], S) < 1e-12


# ---------------------------------------------------------------- recurrence

def test_worked_example_d2(oracle_lib):
    from oracle import oracle as O
    ex = json.load(open(os.path.join(GOLDEN, "worked_example_d2.json")))
    toks = ex["tokens"]
    L = len(toks)
    q = np.array([t["q"] for t in toks]).reshape(1, L, 1, 2)
    k = np.array([t["k"] for t in toks]).reshape(1, L, 1, 2)
    v = np.array([t["v"] for t in toks]).reshape(1, L, 1, 2)
    g = np.log(np.array([t["exp_g"] for t in toks])).reshape(1, L, 1)
    beta = np.array([t["beta"] for t in toks]).reshape(1, L, 1)
    out, S = O.core(q, k, v, g, beta)
    assert np.allclose(out[0, :, 0], ex["expected"]["o"], rtol=0, atol=1e-15)
    assert np.allclose(S[0, 0], ex["expected"]["S_after"][-1], rtol=0, atol=1e-15)
    # first token alone
    out1, S1 = O.core(q[:, :1], k[:, :1], v[:, :1], g[:, :1], beta[:, :1])
    assert np.allclose(S1[0, 0], ex["expected"]["S_after"][0], atol=0)


def rand_features(rng, B, L, Hk, Hv, dk, dv, slow=False):
    q = rng.standard_normal((B, L, Hk, dk))
    k = rng.standard_normal((B, L, Hk, dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, L, Hv, dv))
    g = -rng.uniform(0.0, 0.05 if slow else 3.0, (B, L, Hv))
    beta = rng.uniform(0.0, 1.0, (B, L, Hv))
    S0 = 0.05 * rng.standard_normal((B, Hv, dk, dv))
    return q, k, v, g, beta, S0


def test_first_token_closed_form(oracle_lib):
    """From S = 0: S_1 = beta k v^T and o_1 = beta (k . q) v."""
    from oracle import oracle as O
    rng = np.random.default_rng(3)
    q, k, v, g, beta, _ = rand_features(rng, 1, 1, 1, 1, 16, 12)
    out, S = O.core(q, k, v, g, beta)
    b = beta[0, 0, 0]
    assert np.allclose(S[0, 0], b * np.outer(k[0, 0, 0], v[0, 0, 0]), rtol=1e-15, atol=1e-17)
    assert np.allclose(out[0, 0, 0], b * (k[0, 0, 0] @ q[0, 0, 0]) * v[0, 0, 0], rtol=1e-13,
                       atol=1e-16)


def test_beta_zero_is_pure_decay(oracle_lib):
    """beta = 0: S_t = exp(g_1 + ... + g_t) S_0 and o_t = S_t^T q_t."""
    from oracle import oracle as O
    rng = np.random.default_rng(4)
    q, k, v, g, beta, S0 = rand_features(rng, 1, 20, 1, 2, 8, 8)
    beta[:] = 0.0
    out, S = O.core(q, k, v, g, beta, S0)
    for h in range(2):
        cum = np.cumsum(g[0, :, h])
        assert np.allclose(S[0, h], np.exp(cum[-1]) * S0[0, h], rtol=1e-13)
        for t in range(20):
            assert np.allclose(out[0, t, h], np.exp(cum[t]) * S0[0, h].T @ q[0, t, 0],
                               rtol=1e-12, atol=1e-300)


def test_orthonormal_keys_store_retrieve_overwrite(oracle_lib):
    """g = 0, beta = 1, orthonormal keys: S = sum k_i v_i^T; querying k_j
    returns v_j; writing key k_j again replaces its value."""
    from oracle import oracle as O
    rng = np.random.default_rng(5)
    d = 16
    Qm, _ = np.linalg.qr(rng.standard_normal((d, d)))
    keys = Qm.T                                   # rows orthonormal
    vals = rng.standard_normal((d, d))
    L = d + 3
    k = np.zeros((1, L, 1, d))
    v = np.zeros((1, L, 1, d))
    k[0, :d, 0] = keys
    v[0, :d, 0] = vals
    new = rng.standard_normal((3, d))
    for i, j in enumerate((2, 7, 2)):             # overwrite 2, 7, then 2 again
        k[0, d + i, 0] = keys[j]
        v[0, d + i, 0] = new[i]
    q = k.copy()
    g = np.zeros((1, L, 1))
    beta = np.ones((1, L, 1))
    out, S = O.core(q, k, v, g, beta)
    assert np.allclose(out[0, :d, 0], vals, atol=1e-13)           # read back each write
    assert np.allclose(S[0, 0], keys.T @ np.vstack([vals[:2], [new[2]], vals[3:7], [new[1]],
                                                    vals[8:]]), atol=1e-13)
    for j, want in ((2, new[2]), (7, new[1]), (5, vals[5])):
        assert np.allclose(S[0, 0].T @ keys[j], want, atol=1e-13)


def test_dense_transition_brute_force(oracle_lib):
    """d <= 8: S_t = exp(g)(I - beta k k^T) S_{t-1} + beta k v^T with explicit
    matrices, o_t = S_t^T q_t -- the rule rewritten as a linear system step."""
    from oracle import oracle as O
    rng = np.random.default_rng(6)
    for dk, dv in ((2, 3), (5, 5), (8, 4)):
        q, k, v, g, beta, S0 = rand_features(rng, 2, 30, 1, 2, dk, dv)
        out, S = O.core(q, k, v, g, beta, S0)
        for b in range(2):
            for h in range(2):
                St = S0[b, h].copy()
                for t in range(30):
                    kk = k[b, t, 0][:, None]
                    Tm = np.exp(g[b, t, h]) * (np.eye(dk) - beta[b, t, h] * kk @ kk.T)
                    St = Tm @ St + beta[b, t, h] * kk @ v[b, t, h][None, :]
                    assert np.allclose(out[b, t, h], St.T @ q[b, t, 0], rtol=1e-12, atol=1e-14)
                assert np.allclose(S[b, h], St, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("slow", [False, True])
def test_recurrent_equals_chunked(oracle_lib, slow):
    """The per-token rule and the chunked (chunk 64) form agree in fp64, with a
    ragged last chunk and a nonzero initial state."""
    from oracle import oracle as O
    rng = np.random.default_rng(8 + slow)
    q, k, v, g, beta, S0 = rand_features(rng, 1, 200, 1, 2, 32, 16, slow=slow)
    out, S = O.core(q, k, v, g, beta, S0)
    for chunk in (64, 16):
        oc, Sc = chunked_ref.chunked(q, k, v, g, beta, S0, chunk=chunk)
        assert rel(oc, out) < 1e-12
        assert rel(Sc, S) < 1e-12


def test_split_anywhere_continuation_is_bitwise(oracle_lib):
    """Running L tokens, or L1 then L - L1 from the carried (conv, S) state,
    gives identical bits, including the checkpoints of both halves."""
    from oracle import oracle as O
    w = small_workload(seq_len=40, batch=1)
    x = np_inputs(w)
    full_d = dims_of(w, ckpt_interval=8)
    full = O.layer(full_d, x["qkv"], x["a"], x["b"], x["conv_w"], x["A_log"], x["dt_bias"],
                   x["conv_state"], x["rec_state"], want_ckpt=True)
    ftail, fck = O.conv_tail(full_d, x["qkv"], x["conv_state"], want_ckpt=True)
    for L1 in (1, 2, 5, 8, 17, 39):
        d1 = dims_of(w, ckpt_interval=8)
        d1.seq_len = L1
        p1 = O.layer(d1, x["qkv"][:, :L1], x["a"][:, :L1], x["b"][:, :L1], x["conv_w"],
                     x["A_log"], x["dt_bias"], x["conv_state"], x["rec_state"], want_ckpt=True)
        t1, c1 = O.conv_tail(d1, x["qkv"][:, :L1], x["conv_state"], want_ckpt=True)
        d2 = dims_of(w, ckpt_interval=8, start_pos=L1)
        d2.seq_len = 40 - L1
        p2 = O.layer(d2, x["qkv"][:, L1:], x["a"][:, L1:], x["b"][:, L1:], x["conv_w"],
                     x["A_log"], x["dt_bias"], t1, p1["S"], want_ckpt=True)
        t2, c2 = O.conv_tail(d2, x["qkv"][:, L1:], t1, want_ckpt=True)
        assert np.array_equal(np.concatenate([p1["out"], p2["out"]], axis=1), full["out"])
        assert np.array_equal(p2["S"], full["S"])
        assert np.array_equal(t2, ftail)
        assert np.array_equal(np.concatenate([p1["ckpt_S"], p2["ckpt_S"]]), full["ckpt_S"])
        assert np.array_equal(np.concatenate([c1, c2]), fck)


def test_checkpoint_count_brute_force(oracle_lib):
    from oracle import oracle as O
    for start in (0, 1, 63, 64, 100, 4096):
        for L in (0, 1, 64, 65, 300):
            for iv in (1, 64, 100):
                d = O.Dims(1, L, 1, 1, 2, 2, start_pos=start, ckpt_interval=iv)
                want = sum(1 for p in range(start + 1, start + L + 1) if p % iv == 0)
                assert O.ckpt_count(d) == want


def test_checkpoint_states_match_prefix_runs(oracle_lib):
    """Slot j holds the state after absolute position (j+1)*interval, i.e. the
    final state of a run over just that prefix."""
    from oracle import oracle as O
    w = small_workload(seq_len=30, batch=2)
    x = np_inputs(w)
    d = dims_of(w, ckpt_interval=7)
    full = O.layer(d, x["qkv"], x["a"], x["b"], x["conv_w"], x["A_log"], x["dt_bias"],
                   x["conv_state"], x["rec_state"], want_ckpt=True)
    assert full["ckpt_S"].shape[0] == 4
    for j in range(4):
        p = (j + 1) * 7
        dp = dims_of(w)
        dp.seq_len = p
        pre = O.layer(dp, x["qkv"][:, :p], x["a"][:, :p], x["b"][:, :p], x["conv_w"],
                      x["A_log"], x["dt_bias"], x["conv_state"], x["rec_state"])
        assert np.array_equal(full["ckpt_S"][j], pre["S"])


def test_layer_equals_frontend_then_core_and_head_selection(oracle_lib):
    from oracle import oracle as O
    w = small_workload(seq_len=13)
    x = np_inputs(w)
    d = dims_of(w)
    fe = O.frontend(d, x["qkv"], x["a"], x["b"], x["conv_w"], x["A_log"], x["dt_bias"],
                    x["conv_state"])
    out, S = O.core(fe["q"], fe["k"], fe["v"], fe["g"], fe["beta"], x["rec_state"])
    lay = O.layer(d, x["qkv"], x["a"], x["b"], x["conv_w"], x["A_log"], x["dt_bias"],
                  x["conv_state"], x["rec_state"])
    assert np.array_equal(lay["out"], out) and np.array_equal(lay["S"], S)
    sel = O.layer(d, x["qkv"], x["a"], x["b"], x["conv_w"], x["A_log"], x["dt_bias"],
                  x["conv_state"], x["rec_state"], heads=[3, 0])
    assert np.array_equal(sel["out"][:, :, 0], out[:, :, 3])
    assert np.array_equal(sel["S"][:, 1], S[:, 0])


def test_no_nan_inf_at_extremes(oracle_lib):
    """Gates in their tails (a, b ~ +-30) and zero pre-conv inputs stay finite."""
    from oracle import oracle as O
    w = I.extreme_gates(small_workload(seq_len=20))
    x = np_inputs(w)
    x["qkv"][:, 5:9] = 0
    d = dims_of(w)
    lay = O.layer(d, x["qkv"], x["a"], x["b"], x["conv_w"], x["A_log"], x["dt_bias"],
                  x["conv_state"], x["rec_state"])
    assert np.all(np.isfinite(lay["out"])) and np.all(np.isfinite(lay["S"]))
