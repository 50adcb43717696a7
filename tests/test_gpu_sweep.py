"""Randomised end-to-end sweep of the decode step: many small configurations drawn
from a seeded generator (batch, GQA ratio, head dim, block size, ragged context
length, selector heads / dims / keys per block, key and query formats, p, budgets,
reserved blocks, fp32 or bf16), each run through the three calls and checked against
the oracle (every score, the selection of every row, every output head). Also two
decode steps running concurrently on two streams."""
import math
import random

import pytest
import torch

from block_sparse_long_spot_amd import _lib
from block_sparse_long_spot_amd import workloads as W
from block_sparse_long_spot_amd.decode import DecodeBuffers, decode_step
from test_gpu_parity import run_e2e

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    _lib.load()


def _chunk(fmt):
    return {"int4": 32, "fp4": 32, "int8": 16, "fp8": 16}.get(fmt, 8)


def _configs(n=96, seed=1234):
    rng = random.Random(seed)
    out = []
    while len(out) < n:
        dtype = rng.choice(["f32", "bf16", "bf16"])
        d = rng.choice([64, 128])
        G = rng.choice([1, 2, 4, 8])
        Hkv = rng.choice([1, 2, 4])
        block = rng.choice([16, 32, 64, 128])
        L = rng.randint(1, 40) * block + rng.choice([0, 0, rng.randint(1, block - 1)])
        nb = -(-L // block)
        kf = rng.choice(["f32", "bf16", "int8", "fp8", "int4", "fp4"])
        qf = rng.choice([None, None, "int8", "fp8", "int4", "fp4"])
        d_idx = rng.choice([32, 64, 128])
        H_idx = rng.choice([1, 2, 4, 8, 16])
        if H_idx * d_idx // _chunk(kf) > 64:
            continue
        kpb = rng.choice([1, 1, 2, min(block, 16)])
        n_sink, n_rec = rng.randint(0, 3), rng.randint(0, 4)
        r = min(nb, min(n_sink, nb) + min(n_rec, nb))
        K_max = rng.randint(max(r, 1), nb + 3)
        K_min = rng.randint(0, min(8, K_max))
        p = rng.choice([0.0, 0.3, 0.9, 0.99, 1.0])
        B = rng.randint(1, 3)
        structure = "zipf" if nb - r > 2 and rng.random() < 0.5 else "none"
        out.append(W.Workload(
            f"sweep{len(out)}", B=B, Hq=G * Hkv, Hkv=Hkv, d=d, L=L, block=block, H_idx=H_idx,
            d_idx=d_idx, kpb=kpb, dtype=dtype, sel_k_dtype=kf, p=p, K_min=K_min, K_max=K_max,
            n_sink=n_sink, n_rec=n_rec, structure=structure, zipf_s=rng.choice([1.1, 1.6]),
            seed=1000 + len(out), sel_q_dtype=qf))
    return out


SWEEP = _configs()


@pytest.mark.parametrize("wl", SWEEP, ids=lambda w: w.name)
def test_decode_sweep(wl):
    print(f"{wl.name}: {wl}", flush=True)
    inp = W.make_inputs(wl, device=DEV)
    run_e2e(wl, inp, tag=wl.name)


def test_two_streams_concurrently():
    """Two decode steps with their own buffers on two streams, interleaved: each result
    equals the same step run alone, bit for bit (the library keeps no shared state)."""
    wa = W.WORKLOADS["c2_32k_b4"]
    wb = W.WORKLOADS["c3_128k_b8"].with_(B=2, L=16384)
    ia, ib = W.make_inputs(wa, device=DEV, seed=5), W.make_inputs(wb, device=DEV, seed=6)
    ref = []
    for wl, inp in ((wa, ia), (wb, ib)):
        bufs = DecodeBuffers.of(wl, torch.bfloat16)
        decode_step(inp, wl, bufs)
        torch.cuda.synchronize()
        ref.append((bufs.sel_idx.clone(), bufs.out.clone()))
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    ba = DecodeBuffers.of(wa, torch.bfloat16)
    bb = DecodeBuffers.of(wb, torch.bfloat16)
    for _ in range(20):
        decode_step(ia, wa, ba, stream=sa)
        decode_step(ib, wb, bb, stream=sb)
    torch.cuda.synchronize()
    assert torch.equal(ba.sel_idx, ref[0][0]) and torch.equal(ba.out, ref[0][1])
    assert torch.equal(bb.sel_idx, ref[1][0]) and torch.equal(bb.out, ref[1][1])


def _prefill_configs(n=40, seed=4321):
    rng = random.Random(seed)
    out = []
    for i in range(n):
        Tq = rng.choice([1, 7, 16, 33, 64, 100, 128])
        T = rng.randint(1, 6) * Tq + rng.choice([0, rng.randint(0, max(Tq - 1, 0))])
        q_pos0 = rng.choice([0, 0, rng.randint(1, 700)])
        G, Hkv = rng.choice([1, 2, 4, 8]), rng.choice([1, 2])
        H_idx = rng.choice([1, 2, 4, 8])
        d_idx = rng.choice([32, 64, 128])
        if H_idx * d_idx // 8 > 64:
            H_idx = 4
        out.append(dict(B=rng.randint(1, 2), T=T, Tq=Tq, q_pos0=q_pos0, Hq=G * Hkv, Hkv=Hkv,
                        H_idx=H_idx, d_idx=d_idx, kpb=rng.choice([1, 1, 2, 3]),
                        p=rng.choice([0.0, 0.5, 0.9, 1.0]), K_min=rng.randint(0, 6),
                        n_sink=rng.randint(0, 2), n_rec=rng.randint(0, 4), seed=2000 + i))
    return out


@pytest.mark.parametrize("c", _prefill_configs(), ids=lambda c: f"T{c['T']}-Tq{c['Tq']}-p0{c['q_pos0']}-s{c['seed']}")
def test_prefill_sweep(c):
    """Random whole-sequence prefills (any tile size, start position and GQA ratio)
    against the oracle, every tile."""
    import numpy as np
    from oracle import spot_oracle as O
    from parity import (assert_out_close, assert_scores_close, assert_selection_e2e,
                        assert_topp_unit, gpu_sets, np64, tile_score_magnitude)
    print(c, flush=True)
    B, T, Tq, q_pos0, Hq, Hkv = c["B"], c["T"], c["Tq"], c["q_pos0"], c["Hq"], c["Hkv"]
    H, di, kpb, d, block = c["H_idx"], c["d_idx"], c["kpb"], 128, 64
    L = q_pos0 + T
    nb = -(-L // block)
    n_tiles = -(-T // Tq)
    g = torch.Generator(device=DEV)
    g.manual_seed(c["seed"])
    sel_q = torch.randn(B, T, H, di, generator=g, device=DEV).bfloat16()
    sel_w = torch.randn(B, T, H, generator=g, device=DEV)
    sel_k = torch.randn(B, nb, kpb, H, di, generator=g, device=DEV).bfloat16()
    Q = torch.randn(B, Hq, T, d, generator=g, device=DEV).bfloat16()
    K = torch.randn(B, Hkv, L, d, generator=g, device=DEV).bfloat16()
    V = torch.randn(B, Hkv, L, d, generator=g, device=DEV).bfloat16()
    K_max = max(nb, 1)
    K_min, p, n_sink, n_rec = c["K_min"], c["p"], c["n_sink"], c["n_rec"]
    scores = torch.full((B, n_tiles, nb), float("nan"), device=DEV)
    _lib.spot_prefill_select_score(sel_q, sel_w, sel_k, scores, q_pos0, kpb=kpb, Tq=Tq)
    idx = torch.empty(B, n_tiles, K_max, dtype=torch.int32, device=DEV)
    cnt = torch.empty(B, n_tiles, dtype=torch.int32, device=DEV)
    _lib.spot_prefill_select_topp(scores, idx, cnt, None, p, K_min, K_max, n_sink, n_rec, q_pos0,
                                  T, Tq=Tq)
    out = torch.full((B, Hq, T, d), float("nan"), device=DEV).bfloat16()
    scale = 1 / math.sqrt(d)
    _lib.spot_prefill_attn(Q, K, V, idx, cnt, out, q_pos0, scale, Tq=Tq)
    torch.cuda.synchronize()
    sq, sw, sk, gs = np64(sel_q), np64(sel_w), np64(sel_k), np64(scores)
    Qd, Kd, Vd, got = np64(Q), np64(K), np64(V), np64(out)
    pf = float(np.float32(p))
    for t in range(n_tiles):
        q0, q1 = t * Tq, min((t + 1) * Tq, T)
        nb_t = -(-(q_pos0 + q1) // block)
        ref_s = O.prefill_tile_score(sq[:, q0:q1], sw[:, q0:q1], sk, q_pos0 + q0, block)
        assert_scores_close(gs[:, t, :nb_t], ref_s,
                            tile_score_magnitude(sq[:, q0:q1], sw[:, q0:q1], sk, q_pos0 + q0,
                                                 block))
        sets = gpu_sets(idx[:, t], cnt[:, t])
        for b in range(B):
            assert_topp_unit(sets[b], gs[b, t, :nb_t], pf, K_min, K_max, n_sink, n_rec,
                             tag=f"tile {t} row {b}")
            assert_selection_e2e(sets[b], ref_s[b], pf, K_min, K_max, n_sink, n_rec,
                                 tag=f"tile {t} e2e {b}")
        ref = O.prefill_attention(Qd[:, :, q0:q1], Kd, Vd, sets, block, scale, q_pos0 + q0)
        assert_out_close(got[:, :, q0:q1], ref, torch.bfloat16, tag=f"tile {t}")
