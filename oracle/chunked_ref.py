"""fp64 chunked form of the gated delta rule -- TEST INFRASTRUCTURE ONLY.

A second, structurally different formulation of the recurrence in
``gdn_oracle.c``, used only to pin that oracle (and to debug kernels on the
CPU).  The cortex commit page "feat(stage-8c): linear-attention layer
(Qwen3-Next GatedDeltaNet)" names the chunked algorithm with chunk 64 in its
"Performance note" as a faster evaluation of the same per-token rule
("Delta rule"); the pages print no derivation, so the one used here is
stated in full below and derived from that rule.

Within one chunk of rows r = 1..C with incoming state S0, let
gamma_r = g_1 + ... + g_r and Gamma_r = exp(gamma_r).  Unrolling the rule,

    S_r = Gamma_r S0 + sum_{i<=r} exp(gamma_r - gamma_i) k_i delta_i^T
    delta_r = beta_r (v_r - Gamma_r S0^T k_r
                      - sum_{i<r} exp(gamma_r - gamma_i) (k_r . k_i) delta_i)

so with the strictly lower A[r,i] = beta_r exp(gamma_r - gamma_i) (k_r . k_i)
the chunk's deltas solve (I + A) Delta = diag(beta) V - diag(beta Gamma) K S0.
Then  O = diag(Gamma) Q S0 + (M * Q K^T) Delta  with M[r,i] = exp(gamma_r -
gamma_i) for i <= r (else 0), and the state after the chunk is
S_C = Gamma_C S0 + (diag(exp(gamma_C - gamma)) K)^T Delta.

Only non-positive exponents are ever evaluated (g <= 0).
"""
from __future__ import annotations

import numpy as np


def chunked_head(q, k, v, g, beta, S0=None, chunk=64):
    """One value head.  q, k [L, dk]; v [L, dv]; g, beta [L]; S0 [dk, dv].

    Returns (out [L, dv], S [dk, dv]).  All fp64; the triangular system of
    each chunk is solved with numpy's dense solver (a library primitive).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    g = np.asarray(g, np.float64)
    beta = np.asarray(beta, np.float64)
    L, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, np.float64, copy=True)
    out = np.zeros((L, dv))
    for c0 in range(0, L, chunk):
        c1 = min(L, c0 + chunk)
        Q, K, V = q[c0:c1], k[c0:c1], v[c0:c1]
        bt = beta[c0:c1]
        gam = np.cumsum(g[c0:c1])
        n = c1 - c0
        diff = gam[:, None] - gam[None, :]
        lower_incl = np.tril(np.ones((n, n), bool))
        lower_strict = np.tril(np.ones((n, n), bool), -1)
        M = np.where(lower_incl, np.exp(np.where(lower_incl, diff, 0.0)), 0.0)
        A = np.where(lower_strict, bt[:, None] * M * (K @ K.T), 0.0)
        rhs = bt[:, None] * V - (bt * np.exp(gam))[:, None] * (K @ S)
        Delta = np.linalg.solve(np.eye(n) + A, rhs)
        out[c0:c1] = np.exp(gam)[:, None] * (Q @ S) + (M * (Q @ K.T)) @ Delta
        S = np.exp(gam[-1]) * S + (np.exp(gam[-1] - gam)[:, None] * K).T @ Delta
    return out, S


def chunked(q, k, v, g, beta, S0=None, chunk=64):
    """All heads.  q, k [B, L, Hk, dk]; v [B, L, Hv, dv]; g, beta [B, L, Hv]."""
    B, L, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    r = Hv // Hk
    out = np.zeros((B, L, Hv, dv))
    S = np.zeros((B, Hv, dk, dv))
    for b in range(B):
        for h in range(Hv):
            s0 = None if S0 is None else S0[b, h]
            out[b, :, h], S[b, h] = chunked_head(q[b, :, h // r], k[b, :, h // r], v[b, :, h],
                                                 g[b, :, h], beta[b, :, h], s0, chunk)
    return out, S
