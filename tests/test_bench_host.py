"""Host-side checks of bench.py (no GPU): the one-GPU refusal and the
algorithmic figures the roofline fractions are priced on.

The FLOP count of the chunked form is checked by counting multiply-adds from
explicit masks of each product, and the byte floors by summing the sizes of
the tensors a call must read and write, built as numpy arrays of the right
shape and dtype.  The products are those of the chunked evaluation (chunk 64)
that the cortex commit page "feat(stage-8c): linear-attention layer
(Qwen3-Next GatedDeltaNet)" names in its "Performance note", of the
per-token rule in its "Delta rule" section; the shapes are those of the
"Add Qwen3.6-27B hybrid DeltaNet/GQA contrib model and vLLM serving path"
page ("Validation") and the Qwen3-Coder-Next page ("Model Architecture").
"""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def run_bench(args, extra_env=None):
    env = dict(os.environ)
    env.update(extra_env or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, capture_output=True,
                          text=True, env=env, timeout=120)


def test_bench_refuses_more_than_one_gpu():
    r = run_bench(["--gpus", "2", "--steps", "1", "--warmup", "0"])
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_bench_refuses_a_multi_rank_launch():
    r = run_bench(["--steps", "1"], {"WORLD_SIZE": "2", "RANK": "0"})
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def mac_count(mask: np.ndarray, inner: int) -> int:
    """Multiply-adds of an output whose kept entries are `mask`, each an inner
    product of length `inner`."""
    return int(mask.sum()) * inner


@pytest.mark.parametrize("C,d", [(64, 128), (16, 32), (8, 4)])
def test_prefill_flops_from_product_masks(C, d):
    ones = np.ones((C, C), dtype=bool)
    strict = np.tril(ones, -1)        # K K^T below the diagonal (beta-scaled A)
    incl = np.tril(ones, 0)           # causal products that keep the diagonal
    full_cd = np.ones((C, d), dtype=bool)
    full_dd = np.ones((d, d), dtype=bool)
    macs = mac_count(strict, d)                    # K K^T
    macs += mac_count(incl, d)                     # Q K^T
    # the two T-products (T K and T V: a C x C lower-inclusive matrix times
    # C x d) and P Delta: each output entry (t, j) sums over s <= t
    tri_cd = sum(int(incl[t].sum()) for t in range(C)) * d
    macs += 3 * tri_cd
    macs += mac_count(full_cd, d)                  # W S0
    macs += mac_count(full_cd, d)                  # Q S0
    macs += mac_count(full_dd, C)                  # K^T Delta (d x d, inner C)
    flops = 2 * macs + C ** 3 / 3                  # the triangular solve, as counted by the formula
    assert bench.prefill_flops_per_token_head(C, d) == pytest.approx(flops / C, rel=1e-12)


def nbytes(*arrays) -> int:
    return sum(a.nbytes for a in arrays)


@pytest.mark.parametrize("B,L,Hk,Hv,d", [(1, 16384, 16, 48, 128), (8, 4096, 16, 32, 128), (2, 100, 2, 6, 16)])
def test_prefill_floor_from_tensor_sizes(B, L, Hk, Hv, d):
    bf16, f32 = np.dtype(np.float16), np.dtype(np.float32)   # float16 stands in for bf16's 2 bytes
    conv_dim = 2 * Hk * d + Hv * d
    e = lambda shape, dt: np.empty(shape, dtype=dt)  # noqa: E731
    reads = [e((B, L, conv_dim), bf16), e((B, L, Hv), bf16), e((B, L, Hv), bf16)]   # qkv, a, b
    # o, the final recurrent state and the conv tail (K - 1 = 3 rows)
    writes = [e((B, L, Hv, d), bf16), e((B, Hv, d, d), f32), e((B, 3, conv_dim), bf16)]
    assert bench.prefill_bytes(B, L, Hk, Hv, d) == nbytes(*reads, *writes)
    # with an initial state, it and the initial conv tail are read as well
    initial = [e((B, Hv, d, d), f32), e((B, 3, conv_dim), bf16)]
    assert bench.prefill_bytes(B, L, Hk, Hv, d, state_in=True) == nbytes(*reads, *writes, *initial)
    assert bench.varlen_bytes(B * L, B, Hk, Hv, d) == nbytes(*reads, *writes, *initial)


@pytest.mark.parametrize("B,Hk,Hv,d", [(32, 16, 48, 128), (8, 16, 32, 128), (3, 2, 6, 16)])
def test_decode_bytes_from_tensor_sizes(B, Hk, Hv, d):
    bf16, f32 = np.dtype(np.float16), np.dtype(np.float32)
    conv_dim = 2 * Hk * d + Hv * d
    e = lambda shape, dt: np.empty(shape, dtype=dt)  # noqa: E731
    tensors = [
        e((B, Hv, d, d), f32), e((B, Hv, d, d), f32),          # recurrent state read and written
        e((B, conv_dim), bf16),                                # this token's qkv
        e((B, 3, conv_dim), bf16), e((B, 3, conv_dim), bf16),  # conv tail in and out
        e((B, Hv, d), bf16),                                   # o
        e((B, Hv), bf16), e((B, Hv), bf16),                    # a, b
        e((conv_dim, 4), bf16),                                # conv taps
        e((Hv,), f32), e((Hv,), f32),                          # A_log, dt_bias
    ]
    assert bench.decode_bytes(B, Hk, Hv, d) == nbytes(*tensors)
