"""The bf16 output bound used by the GPU parity tests, checked on the CPU at the shape of
the 128K decode workloads (one query, one KV head with its 4 query heads, 256 selected
64-token blocks out of 2048, d = 128, N(0,1) data).

A numpy model of the decode kernel's arithmetic (scores in fp32 from bf16 inputs, a
per-run online softmax, probabilities rounded to bf16 for P.V, fp32 row sums of the
unrounded probabilities, runs merged in fp32, the output rounded to bf16) must pass the
bound against the oracle; the same model with one of the four 64-block runs of the
batch-8 split plan left out must fail it. The plain 2e-2 absolute check cannot tell the
two apart at this size: every output element is a weighted mean of 16384 values, about
0.01 in size. No GPU needed.
"""
import math

import numpy as np
import pytest
import torch

from oracle import spot_oracle as O
from parity import (BF16_U, assert_bf16_rounding_bound, assert_out_close, attention_magnitude,
                    bf16_attention_bound)

L, BLOCK, D, G, NSEL, NRUN = 131072, 64, 128, 4, 256, 4


def bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16) \
        .float().numpy()


@pytest.fixture(scope="module")
def case():
    g = torch.Generator().manual_seed(2024)
    nb = L // BLOCK
    sel = sorted(torch.randperm(nb, generator=g)[:NSEL].tolist())
    tok = np.concatenate([np.arange(b * BLOCK, (b + 1) * BLOCK) for b in sel])
    q = bf16(torch.randn(1, G, D, generator=g).numpy())
    K = np.zeros((1, 1, L, D), np.float32)
    V = np.zeros((1, 1, L, D), np.float32)
    K[0, 0, tok] = bf16(torch.randn(len(tok), D, generator=g).numpy())
    V[0, 0, tok] = bf16(torch.randn(len(tok), D, generator=g).numpy())
    scale = 1.0 / math.sqrt(D)
    ref = O.sparse_attention(q, K, V, [sel], BLOCK, scale)
    mag = attention_magnitude(q, K, V, [sel], BLOCK, scale, [(0, h) for h in range(G)])
    return dict(sel=sel, q=q, K=K, V=V, scale=scale, ref=ref,
                mag=[mag[(0, h)] for h in range(G)])


def kernel_model(c, drop_run=None):
    """The decode kernel's arithmetic on the CPU, runs of NSEL / NRUN blocks."""
    sel, q, K, V = c["sel"], c["q"][0], c["K"][0, 0], c["V"][0, 0]
    qs = np.float32(c["scale"] * 1.4426950408889634)
    per = NSEL // NRUN
    parts = []
    for r in range(NRUN):
        if r == drop_run:
            continue
        tok = np.concatenate([np.arange(b * BLOCK, (b + 1) * BLOCK)
                              for b in sel[r * per:(r + 1) * per]])
        z = (K[tok] @ q.T).astype(np.float32) * qs                  # [tokens][G], log2 units
        m = z.max(axis=0)
        p = np.exp2(z - m).astype(np.float32)
        l = p.sum(axis=0, dtype=np.float32)
        acc = (bf16(p).T @ V[tok]).astype(np.float32)              # P in bf16 on the MFMA
        parts.append((m, l, acc))
    M = np.max([m for m, _, _ in parts], axis=0)
    num = sum(np.exp2(m - M)[:, None] * acc for m, _, acc in parts)
    den = sum(np.exp2(m - M) * l for m, l, _ in parts)
    return bf16(num / den[:, None])[None]


def test_bound_holds_for_the_kernel_arithmetic(case):
    got = kernel_model(case)
    assert_out_close(got, case["ref"], torch.bfloat16, tag="model", mag=case["mag"])
    # the bound is a few times the actual error, not orders of magnitude above it
    err = np.abs(got - case["ref"])[0]
    bounds = np.stack([bf16_attention_bound(A, S, ez, case["ref"][0, h])
                       for h, (A, S, ez) in enumerate(case["mag"])])
    assert (err < bounds).all()
    assert bounds.max() < 20 * err.max()
    # far below the worst case u * A, which cannot see a single dropped block here
    worst = np.stack([BF16_U * A for A, _, _ in case["mag"]])
    assert bounds.max() < 0.5 * worst.min()


@pytest.mark.parametrize("run", range(NRUN))
def test_bound_catches_a_dropped_run(case, run):
    got = kernel_model(case, drop_run=run)
    # the stated 2e-2 absolute tolerance alone lets the truncated sum through in some of
    # the heads (each head's largest change is 0.017 ... 0.028 here)
    per_head = np.abs(got - case["ref"])[0].max(axis=-1)
    assert per_head.min() <= 2e-2
    # every one of the four heads sees it on its own
    for h in range(G):
        with pytest.raises(AssertionError, match="rounding bound"):
            assert_bf16_rounding_bound(got[:, h], case["ref"][:, h], [case["mag"][h]],
                                       tag=f"head {h}")


def test_bound_catches_a_dropped_block(case):
    """Finer than a run: one 64-token block of the 256 left out."""
    c = dict(case)
    c["sel"] = case["sel"][:100] + case["sel"][101:]
    got = kernel_model(c)
    assert np.abs(got - case["ref"]).max() <= 2e-2
    with pytest.raises(AssertionError, match="rounding bound"):
        assert_out_close(got, case["ref"], torch.bfloat16, tag="dropped block", mag=case["mag"])
