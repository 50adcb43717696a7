"""GPU parity: every C entry point against the CPU oracle on the same seeded inputs.

Small and ragged cases cover several tiles and every supported shape; the five
workloads run end to end, the 128K ones at full size in the launch configuration the
benchmark times (the split plan is a function of the sizes only), with outputs
compared on sampled rows.
"""
import math
import random

import numpy as np
import pytest
import torch

from block_sparse_long_spot_amd import _lib
from block_sparse_long_spot_amd import workloads as W
from block_sparse_long_spot_amd.decode import DecodeBuffers, DecodeStep, decode_step
from oracle import spot_oracle as O
from parity import (assert_out_close, assert_scores_close, assert_selection_e2e,
                    assert_topp_unit, attention_magnitude, decode_selector, decoded_keys,
                    decoded_query, gpu_sets, np64, score_magnitude)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def log(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    _lib.load()   # raises when libspot.so is missing: no fallback exists


def cpu_gen(seed):
    return torch.Generator().manual_seed(seed)


# ------------------------------------------------------------------ spot_select_score
SCORE_CASES = [
    # B, nb, kpb, H, d_idx, query format, key format
    (1, 64, 1, 4, 32, "f32", "f32"),
    (3, 333, 1, 4, 64, "bf16", "bf16"),
    (2, 1000, 1, 4, 64, "f32", "bf16"),
    (2, 77, 3, 2, 128, "bf16", "bf16"),
    (2, 130, 16, 4, 128, "bf16", "bf16"),
    (1, 50, 1, 8, 32, "f32", "f32"),
    (2, 300, 1, 16, 32, "bf16", "f32"),
    (1, 9, 2, 1, 64, "f32", "f32"),
    (2, 257, 1, 4, 64, "bf16", "int4"),
    (2, 65, 4, 4, 64, "f32", "int4"),
    (1, 100, 1, 2, 128, "bf16", "int4"),
    (1, 31, 1, 16, 32, "f32", "int4"),
    (2, 2048, 1, 4, 64, "bf16", "bf16"),
    # 8-bit and FP4 key caches, and quantised queries (§5.3, Appendix G)
    (2, 257, 1, 4, 64, "bf16", "int8"),
    (2, 65, 5, 4, 64, "int8", "int8"),
    (1, 40, 1, 16, 32, "bf16", "int8"),
    (2, 300, 1, 4, 64, "bf16", "fp8"),
    (2, 65, 3, 4, 64, "fp8", "fp8"),
    (1, 70, 1, 8, 128, "f32", "fp8"),
    (2, 257, 1, 4, 64, "bf16", "fp4"),
    (1, 100, 1, 2, 128, "f32", "fp4"),
    (1, 130, 16, 4, 128, "fp4", "fp4"),
    (1, 40, 1, 64, 32, "bf16", "fp4"),
    (2, 77, 1, 4, 64, "int4", "int4"),
    (1, 31, 1, 16, 32, "fp8", "f32"),
    (2, 50, 2, 4, 64, "int4", "bf16"),
    (2, 2048, 1, 4, 64, "bf16", "fp4"),
    # one key per block on grids of 2048 and 4096+ one-round work-groups, so each lane
    # scores 2 or 4 blocks, with the last round ragged (nb not a multiple of a
    # work-group's blocks)
    (8, 2047, 1, 4, 64, "bf16", "bf16"),
    (16, 2050, 1, 4, 64, "f32", "bf16"),
    (64, 2049, 1, 4, 64, "bf16", "int4"),
    (32, 1029, 1, 4, 64, "bf16", "fp8"),
]


@pytest.mark.parametrize("case", SCORE_CASES, ids=lambda c: "-".join(map(str, c)))
def test_select_score_parity(case):
    B, nb, kpb, H, di, qf, kf = case
    log(f"score case {case}")
    g = cpu_gen(nb * 7 + kpb + len(qf) + 3 * len(kf))
    sel_q, q_scale = W.quantize_selector(torch.randn(B, H, di, generator=g), qf)
    sel_w = torch.randn(B, H, generator=g)            # signed weights
    sel_k, k_scale = W.quantize_selector(torch.randn(B, nb, kpb, H, di, generator=g), kf)
    dev = lambda t: None if t is None else t.to(DEV)
    scores = torch.full((B, nb), float("nan"), device=DEV)
    _lib.spot_select_score(dev(sel_q), sel_w.to(DEV), dev(sel_k), dev(k_scale), scores, kpb=kpb,
                           sel_q_scale=dev(q_scale))
    torch.cuda.synchronize()
    qdec = decode_selector(sel_q, q_scale)
    keys = decode_selector(sel_k, k_scale)
    ref = O.select_score(qdec, np64(sel_w), keys)
    assert_scores_close(np64(scores), ref, score_magnitude(qdec, np64(sel_w), keys))


# ------------------------------------------------------------------ spot_select_topp
def _topp_rows(kind, B, nb, g):
    if kind == "normal":
        return torch.randn(B, nb, generator=g) * 3
    if kind == "wide":
        return torch.randn(B, nb, generator=g) * 30
    if kind == "ties":
        return torch.round(torch.randn(B, nb, generator=g) * 2) / 2
    if kind == "flat":
        return torch.zeros(B, nb)
    if kind == "signed_zero":
        x = torch.round(torch.randn(B, nb, generator=g))
        x[x == 0] = -0.0
        x[:, ::3] = 0.0
        return x
    if kind.startswith("tiebin"):
        # 10 high blocks, then a group of n equal scores where the cut falls, then noise
        n = int(kind[6:])
        x = torch.rand(B, nb, generator=g) - 2.0
        x[:, 5:15] = 4.0
        x[:, 20:20 + n] = 2.5
        return x
    if kind.startswith("nearbin"):
        # 10 high blocks, then n blocks within 1/64 of a unit of each other where the cut
        # falls (distinct scores in random order, pairs of them tied), then noise
        n = int(kind[7:])
        x = torch.rand(B, nb, generator=g) - 2.0
        x[:, 5:15] = 4.0
        for r in range(B):
            x[r, 20:20 + n] = 2.49 + torch.div(torch.randperm(n, generator=g), 2,
                                              rounding_mode="floor").float() * 1e-4
        return x
    if kind == "zipf":
        ranks = torch.stack([torch.randperm(nb, generator=g) for _ in range(B)]).float() + 1
        return 1.1 * torch.log(nb / ranks)
    raise ValueError(kind)


TOPP_CASES = [
    # nb, kind, p, K_min, K_max, n_sink, n_rec
    (1, "normal", 0.9, 0, 1, 0, 0),
    (3, "normal", 0.9, 0, 3, 1, 1),
    (7, "ties", 0.5, 2, 7, 1, 1),
    (64, "normal", 0.9, 4, 16, 1, 2),
    (64, "ties", 0.0, 10, 10, 1, 2),
    (100, "wide", 0.95, 0, 100, 2, 3),
    (255, "signed_zero", 0.7, 5, 200, 1, 4),
    (256, "flat", 0.9, 4, 256, 1, 4),
    (257, "normal", 1.0, 0, 257, 1, 4),
    (512, "normal", 0.95, 16, 128, 1, 4),
    (512, "zipf", 0.95, 16, 512, 1, 4),
    (1000, "ties", 0.9, 0, 1000, 0, 0),
    (2048, "zipf", 0.95, 16, 256, 1, 4),
    (2048, "normal", 0.95, 16, 256, 1, 4),
    (2048, "wide", 0.3, 0, 2048, 1, 4),
    (3000, "normal", 0.8, 32, 3000, 8, 16),
    (4096, "zipf", 0.9, 0, 4096, 1, 4),
    (5000, "ties", 0.95, 16, 600, 1, 4),
    (8192, "zipf", 0.9, 32, 8192, 8, 16),
    (12000, "normal", 0.95, 32, 1000, 8, 16),
    (16384, "zipf", 0.95, 32, 16384, 8, 16),
    (200, "tiebin64", 0.9, 0, 200, 1, 2),       # 64 tied blocks at the cut: one-wave rank
    (200, "tiebin65", 0.9, 0, 200, 1, 2),       # 65 tied blocks: exact radix fallback
    (300, "tiebin65", 0.9, 0, 40, 1, 2),        # fallback, then the cap inside the bin
    (300, "tiebin64", 0.5, 30, 300, 1, 2),      # floor lands inside the tied bin
    (200, "nearbin8", 0.9, 0, 200, 1, 2),       # 8 near blocks at the cut: every wave ranks
    (200, "nearbin9", 0.9, 0, 200, 1, 2),       # 9: ranking split over the waves
    (300, "nearbin40", 0.8, 0, 300, 1, 2),      # the nucleus cut inside the bin
    (300, "nearbin40", 0.0, 30, 30, 0, 0),      # a count cut inside the bin
    (300, "nearbin63", 0.9, 16, 40, 1, 2),      # the cap inside the bin
    (40, "normal", 0.9, 100, 40, 1, 2),         # floor above nb
    (10, "normal", 0.9, 0, 10, 6, 6),           # empty residual
    (20, "normal", -0.5, 3, 20, 1, 1),          # p <= 0: floor only
    (20, "normal", 1.7, 0, 8, 1, 1),            # p >= 1: cap binds
    # static top-K (Eq. 6): p <= 0, no reserved blocks, K_min = K_max = K
    (2048, "zipf", 0.0, 1024, 1024, 0, 0),
    (2048, "ties", 0.0, 1024, 1024, 0, 0),
    (8192, "normal", 0.0, 4096, 4096, 0, 0),
    (300, "tiebin65", 0.0, 25, 25, 0, 0),       # K-th block inside a dense tied bin
]


@pytest.mark.parametrize("case", TOPP_CASES, ids=lambda c: "-".join(map(str, c)))
def test_select_topp_parity(case):
    nb, kind, p, K_min, K_max, n_sink, n_rec = case
    log(f"topp case {case}")
    B = 4
    g = cpu_gen(nb * 13 + int(abs(p) * 100))
    scores = _topp_rows(kind, B, nb, g).float().contiguous()
    sd = scores.to(DEV)
    sel_idx = torch.full((B, K_max), 12345, dtype=torch.int32, device=DEV)
    sel_cnt = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    sel_mass = torch.full((B,), -1.0, device=DEV)
    _lib.spot_select_topp(sd, sel_idx, sel_cnt, sel_mass, p, K_min, K_max, n_sink, n_rec)
    torch.cuda.synchronize()
    sets = gpu_sets(sel_idx, sel_cnt)
    pf = float(np.float32(p))
    masses = sel_mass.cpu().numpy()
    for b in range(B):
        row = scores[b].double().numpy()
        assert_topp_unit(sets[b], row, pf, K_min, K_max, n_sink, n_rec, tag=f"row {b}")
        sel, info = O.select_topp_row(row, pf, K_min, K_max, n_sink, n_rec)
        if sets[b] == sel and info["n_res"] > 0:
            assert abs(masses[b] - info["mass"]) <= 1e-6, (masses[b], info["mass"])


@pytest.mark.parametrize("nb,K,kind", [(2048, 1024, "zipf"), (2048, 1024, "ties"),
                                       (777, 100, "flat"), (16384, 8192, "normal")])
def test_static_topk_matches_sort(nb, K, kind):
    """Eq. 6 directly: the K largest scores, ties to the lower block index, by a full
    sort of the GPU's input scores (no top-p machinery on the reference side)."""
    B = 3
    g = cpu_gen(nb + K)
    x = _topp_rows(kind, B, nb, g).float().contiguous()
    scores = x.to(DEV)
    idx = torch.empty(B, K, dtype=torch.int32, device=DEV)
    cnt = torch.empty(B, dtype=torch.int32, device=DEV)
    _lib.spot_select_topp(scores, idx, cnt, None, 0.0, K, K, 0, 0)
    torch.cuda.synchronize()
    xs = x.numpy().astype(np.float32)
    for b in range(B):
        order = np.lexsort((np.arange(nb), -xs[b].astype(np.float64)))
        want = sorted(order[:K].tolist())
        assert int(cnt[b]) == K
        assert idx[b].cpu().tolist() == want, f"row {b}"


def test_select_topp_deterministic():
    g = cpu_gen(99)
    scores = (torch.randn(8, 2048, generator=g) * 4).to(DEV)
    outs = []
    for _ in range(3):
        idx = torch.empty(8, 256, dtype=torch.int32, device=DEV)
        cnt = torch.empty(8, dtype=torch.int32, device=DEV)
        _lib.spot_select_topp(scores, idx, cnt, None, 0.95, 16, 256, 1, 4)
        outs.append((idx.cpu(), cnt.cpu()))
    for o in outs[1:]:
        assert torch.equal(o[0], outs[0][0]) and torch.equal(o[1], outs[0][1])


# ------------------------------------------------------------------ spot_sparse_attn
ATTN_CASES = [
    # B, Hq, Hkv, d, L, K_max, dtype, pattern
    (1, 8, 2, 64, 4096, 16, "f32", "random"),
    (2, 8, 8, 128, 1000, 9, "f32", "random"),
    (1, 16, 2, 64, 4000, 40, "f32", "ragged_last"),
    (2, 8, 2, 128, 777, 13, "bf16", "ragged_last"),
    (3, 32, 8, 128, 8192, 64, "bf16", "random"),
    (2, 4, 4, 128, 3000, 30, "bf16", "random"),
    (2, 8, 4, 64, 2500, 17, "bf16", "random"),
    (1, 16, 2, 128, 5000, 33, "bf16", "random"),
    (2, 8, 1, 64, 640, 10, "bf16", "all"),
    (2, 32, 8, 128, 4096, 64, "bf16", "invalid_entries"),
    (3, 8, 2, 64, 1024, 8, "f32", "empty_rows"),
    (3, 32, 8, 128, 1024, 8, "bf16", "empty_rows"),
    (1, 32, 8, 128, 70, 2, "bf16", "all"),
    (4, 32, 8, 128, 20000, 256, "bf16", "random"),
    # more than 32 partial slots per (query, head): the slot-by-slot merge (per-query
    # runs at batch 1, runs cut across queries at batch 2 and 3, fp32 runs)
    (1, 8, 1, 128, 13000, 200, "bf16", "random"),
    (2, 8, 1, 64, 13000, 200, "bf16", "skewed"),
    (3, 16, 2, 128, 19300, 300, "bf16", "random"),
    (1, 4, 1, 64, 17000, 256, "f32", "random"),
]


def _sets_for(pattern, B, nb, K_max, g):
    sets = []
    for b in range(B):
        if pattern == "all":
            s = list(range(min(nb, K_max)))
        elif pattern == "ragged_last":
            c = int(torch.randint(1, K_max + 1, (1,), generator=g))
            s = sorted(set(torch.randperm(nb - 1, generator=g)[: c - 1].tolist()) | {nb - 1})
        elif pattern == "empty_rows":
            s = [] if b % 2 == 0 else sorted(torch.randperm(nb, generator=g)[:K_max].tolist())
        elif pattern == "one_long":  # one full row, then rows of 0 to 3 entries, so that
            # a run of the batch-wide cut spans several queries (some of them empty)
            c = min(K_max if b == 0 else (0, 1, 2, 1, 3)[b % 5], K_max, nb)
            s = sorted(torch.randperm(nb, generator=g)[:c].tolist())
        elif pattern == "heavy":  # heavy-tailed counts: many short rows, some empty
            u = float(torch.rand(1, generator=g))
            c = 0 if u < 0.2 else max(1, int(min(nb, K_max) * u ** 3))
            s = sorted(torch.randperm(nb, generator=g)[:c].tolist())
        elif pattern == "skewed":   # a few full rows, the rest short or empty
            c = min(K_max if b % 5 == 0 else (0 if b % 7 == 3 else 1 + b % 4), K_max, nb)
            s = sorted(torch.randperm(nb, generator=g)[:c].tolist())
        else:
            c = int(torch.randint(1, K_max + 1, (1,), generator=g))
            s = sorted(torch.randperm(nb, generator=g)[:c].tolist())
        sets.append(s)
    return sets


@pytest.mark.parametrize("case", ATTN_CASES, ids=lambda c: "-".join(map(str, c)))
def test_sparse_attn_parity(case):
    B, Hq, Hkv, d, L, K_max, dt, pattern = case
    _attn_case(B, Hq, Hkv, d, L, 64, K_max, dt, pattern, tag=str(case))


ATTN_BLOCK_CASES = [
    # B, Hq, Hkv, d, L, block, K_max, dtype, pattern
    (1, 32, 8, 128, 4096, 16, 200, "bf16", "random"),
    (2, 8, 2, 64, 1000, 16, 40, "bf16", "ragged_last"),     # last block of 8 tokens
    (2, 8, 2, 128, 777, 32, 13, "bf16", "ragged_last"),
    (2, 16, 4, 128, 5000, 128, 30, "bf16", "random"),
    (1, 8, 8, 64, 300, 128, 3, "bf16", "all"),              # a chunk wholly past L
    (3, 32, 8, 128, 2048, 16, 64, "bf16", "invalid_entries"),
    (3, 8, 2, 128, 1024, 32, 8, "bf16", "empty_rows"),
    (2, 8, 1, 128, 3000, 16, 7, "bf16", "random"),          # G = 8
    (2, 8, 2, 64, 1500, 16, 50, "f32", "random"),
    (2, 8, 2, 128, 1000, 128, 6, "f32", "ragged_last"),
    (2, 4, 4, 64, 900, 32, 20, "f32", "random"),
    # runs cut across queries: the largest batch that uses them, and the next one up
    # (per-query runs); many short rows beside long ones
    (64, 8, 2, 128, 4096, 64, 40, "bf16", "random"),
    (65, 8, 2, 128, 4096, 64, 40, "bf16", "random"),
    (16, 8, 1, 64, 8192, 16, 300, "bf16", "skewed"),
    (8, 16, 4, 128, 8192, 32, 200, "bf16", "skewed"),
    (4, 8, 2, 128, 8192, 64, 128, "bf16", "invalid_prefix"),
    # runs of a few entries, each spanning up to five queries (the full first row takes
    # ~26 of its 32 slots)
    (8, 32, 8, 128, 8192, 64, 128, "bf16", "one_long"),
    (16, 8, 2, 128, 4096, 16, 64, "bf16", "one_long"),
    (12, 8, 2, 64, 8192, 32, 256, "bf16", "one_long"),
    # longest runs of the split plan: 16 chunks per wave (64 list entries at block 16)
    (4, 8, 8, 64, 32768, 16, 2048, "bf16", "random"),
    (8, 8, 8, 64, 16384, 32, 512, "bf16", "random"),
    (8, 8, 8, 64, 16384, 128, 128, "bf16", "all"),
]


@pytest.mark.parametrize("case", ATTN_BLOCK_CASES, ids=lambda c: "-".join(map(str, c)))
def test_sparse_attn_block_sizes(case):
    B, Hq, Hkv, d, L, block, K_max, dt, pattern = case
    _attn_case(B, Hq, Hkv, d, L, block, K_max, dt, pattern, tag=str(case), dirty_ws=True)


def _flat_configs(n=32, seed=777):
    """Seeded bf16 attention cases at batch 2..48 (runs cut from the batch's lists laid end
    to end, which may span queries), with uneven counts and a dirty workspace."""
    import random
    rng = random.Random(seed)
    out = []
    while len(out) < n:
        B = rng.randint(2, 48)
        Hkv, G = rng.choice([1, 2, 4, 8]), rng.choice([1, 2, 4, 8])
        d, block = rng.choice([64, 128]), rng.choice([16, 32, 64, 128])
        L = rng.randint(2, 120) * block + rng.choice([0, rng.randint(1, block - 1)])
        nb = -(-L // block)
        K_max = rng.randint(1, nb)
        if B * G * Hkv * K_max * block > (1 << 22):
            continue
        out.append((B, G * Hkv, Hkv, d, L, block, K_max, "bf16",
                    rng.choice(["heavy", "heavy", "one_long", "skewed", "random"])))
    return out


@pytest.mark.parametrize("case", _flat_configs(), ids=lambda c: "-".join(map(str, c)))
def test_sparse_attn_flat_sweep(case):
    B, Hq, Hkv, d, L, block, K_max, dt, pattern = case
    _attn_case(B, Hq, Hkv, d, L, block, K_max, dt, pattern, tag=str(case), dirty_ws=True)


def _attn_case(B, Hq, Hkv, d, L, block, K_max, dt, pattern, tag, dirty_ws=False):
    log(f"attn case {tag}")
    g = cpu_gen(L + d + K_max + (block if block != 64 else 0))
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    q = torch.randn(B, Hq, d, generator=g).to(tdt)
    K = torch.randn(B, Hkv, L, d, generator=g).to(tdt)
    V = torch.randn(B, Hkv, L, d, generator=g).to(tdt)
    nb = -(-L // block)
    sets = _sets_for(pattern, B, nb, K_max, g)
    idx = torch.full((B, K_max), -1, dtype=torch.int32)
    cnt = torch.zeros(B, dtype=torch.int32)
    for b, s in enumerate(sets):
        idx[b, : len(s)] = torch.tensor(s, dtype=torch.int32)
        cnt[b] = len(s)
    if pattern == "invalid_prefix":    # whole runs of ignored entries before valid ones
        for b in range(B):
            c = int(cnt[b])
            idx[b, : c // 2] = -1
    if pattern == "invalid_entries":   # out-of-range entries inside the count are ignored
        for b in range(B):
            c = int(cnt[b])
            if c < K_max:
                idx[b, c] = nb + 5
                cnt[b] = c + 1
            idx[b, 0] = -1
    scale = 1.0 / math.sqrt(d)
    out = torch.full((B, Hq, d), float("nan"), device=DEV).to(tdt)
    # workspace contents on entry do not matter: optionally start from all-NaN bytes
    ws = torch.full((_lib.spot_sparse_attn_workspace_bytes(B, Hq, Hkv, d, K_max, block, tdt),),
                    255 if dirty_ws else 0, dtype=torch.uint8, device=DEV)
    idx_d, cnt_d = idx.to(DEV), cnt.to(DEV)
    _lib.spot_sparse_attn(q.to(DEV), K.to(DEV), V.to(DEV), idx_d, cnt_d, out, ws, scale,
                          block=block)
    torch.cuda.synchronize()
    used = [[int(x) for x in idx[b, : int(cnt[b])]] for b in range(B)]
    ref = O.sparse_attention(np64(q), np64(K), np64(V), used, block, scale)
    mag = _magnitudes(q, K, V, used, block, scale) if tdt == torch.bfloat16 else None
    assert_out_close(np64(out), ref, tdt, tag=tag, mag=mag)


def _magnitudes(q, K, V, used, block, scale, rows=None):
    """(A, S, ez) of every (b, hq) row in order, for the bf16 rounding bound."""
    B, Hq = q.shape[0], q.shape[1]
    rows = [(b, h) for b in range(B) for h in range(Hq)] if rows is None else rows
    m = attention_magnitude(q.float(), K, V, used, block, scale, rows)
    return [m[r] for r in rows]


def _batch_sweep(n=24, seed=4321):
    """Seeded attention-only configurations at batch 2..64 (runs cut for the whole
    batch): GQA ratio, head dim, block size, ragged L, K_max, and per-row counts drawn
    from one of several spreads (equal, uniform, a few long rows among short or empty
    ones), sometimes with ignored entries inside the count."""
    rng = random.Random(seed)
    out = []
    while len(out) < n:
        B = rng.choice([2, 3, 5, 8, 13, 32, 64])
        Hkv = rng.choice([1, 2, 4, 8])
        G = rng.choice([1, 2, 4, 8])
        d = rng.choice([64, 128])
        block = rng.choice([16, 32, 64, 128])
        L = rng.randint(2, 64) * block - rng.choice([0, rng.randint(0, block - 1)])
        if B * Hkv * G * L > 2_000_000:
            continue
        nb = -(-L // block)
        K_max = rng.randint(1, nb)
        spread = rng.choice(["equal", "uniform", "skew", "skew_empty"])
        invalid = rng.random() < 0.25
        out.append((len(out), B, G * Hkv, Hkv, d, L, block, K_max, spread, invalid))
    return out


@pytest.mark.parametrize("case", _batch_sweep(), ids=lambda c: "sweep%d" % c[0])
def test_sparse_attn_batch_sweep(case):
    i, B, Hq, Hkv, d, L, block, K_max, spread, invalid = case
    log(f"attn batch sweep {case}")
    g = cpu_gen(9000 + i)
    rng = random.Random(9000 + i)
    q = torch.randn(B, Hq, d, generator=g).bfloat16()
    K = torch.randn(B, Hkv, L, d, generator=g).bfloat16()
    V = torch.randn(B, Hkv, L, d, generator=g).bfloat16()
    nb = -(-L // block)
    idx = torch.full((B, K_max), -1, dtype=torch.int32)
    cnt = torch.zeros(B, dtype=torch.int32)
    for b in range(B):
        if spread == "equal":
            c = K_max
        elif spread == "uniform":
            c = rng.randint(1, K_max)
        else:
            c = K_max if rng.random() < 0.2 else rng.randint(0 if spread == "skew_empty" else 1,
                                                             max(1, K_max // 8))
        s = sorted(torch.randperm(nb, generator=g)[:c].tolist())
        idx[b, :c] = torch.tensor(s, dtype=torch.int32)
        if invalid and c > 1:
            idx[b, rng.randrange(c)] = rng.choice([-3, nb, nb + 7])
        cnt[b] = c
    scale = 1.0 / math.sqrt(d)
    out = torch.full((B, Hq, d), float("nan"), device=DEV).bfloat16()
    ws = torch.full((_lib.spot_sparse_attn_workspace_bytes(B, Hq, Hkv, d, K_max, block),), 255,
                    dtype=torch.uint8, device=DEV)
    _lib.spot_sparse_attn(q.to(DEV), K.to(DEV), V.to(DEV), idx.to(DEV), cnt.to(DEV), out, ws,
                          scale, block=block)
    torch.cuda.synchronize()
    used = [[int(x) for x in idx[b, : int(cnt[b])]] for b in range(B)]
    ref = O.sparse_attention(np64(q), np64(K), np64(V), used, block, scale)
    assert_out_close(np64(out), ref, torch.bfloat16, tag=str(case),
                     mag=_magnitudes(q, K, V, used, block, scale))


def test_sparse_attn_deterministic():
    g = cpu_gen(5)
    B, Hq, Hkv, d, L, K_max = 2, 32, 8, 128, 16384, 64
    q = torch.randn(B, Hq, d, generator=g).bfloat16().to(DEV)
    K = torch.randn(B, Hkv, L, d, generator=g).bfloat16().to(DEV)
    V = torch.randn(B, Hkv, L, d, generator=g).bfloat16().to(DEV)
    idx = torch.stack([torch.randperm(256, generator=g)[:K_max].sort().values
                       for _ in range(B)]).int().to(DEV)
    cnt = torch.full((B,), K_max, dtype=torch.int32, device=DEV)
    ws = torch.zeros(_lib.spot_sparse_attn_workspace_bytes(B, Hq, Hkv, d, K_max), dtype=torch.uint8,
                     device=DEV)
    outs = []
    for _ in range(3):
        out = torch.empty(B, Hq, d, dtype=torch.bfloat16, device=DEV)
        _lib.spot_sparse_attn(q, K, V, idx, cnt, out, ws, 1 / math.sqrt(d))
        outs.append(out.cpu())
    assert all(torch.equal(o, outs[0]) for o in outs[1:])


# ------------------------------------------------------------------ end to end
def run_e2e(wl, inp_dev, check_rows=None, tag=""):
    """Run the three calls, then check scores, selection and (sampled) outputs."""
    B = inp_dev["q"].shape[0]
    dt = inp_dev["q"].dtype
    bufs = DecodeBuffers.of(wl, dt, B=B)
    decode_step(inp_dev, wl, bufs)
    torch.cuda.synchronize()
    log(f"{tag}: GPU step done")
    keys = decoded_keys(inp_dev)
    qdec = decoded_query(inp_dev)
    ref_scores = O.select_score(qdec, np64(inp_dev["sel_w"]), keys)
    assert_scores_close(np64(bufs.scores), ref_scores,
                        score_magnitude(qdec, np64(inp_dev["sel_w"]), keys))
    sets = gpu_sets(bufs.sel_idx, bufs.sel_cnt)
    pf = float(np.float32(wl.p))
    for b in range(B):
        assert_selection_e2e(sets[b], ref_scores[b], pf, wl.K_min, wl.K_max, wl.n_sink,
                             wl.n_rec, tag=f"{tag} row {b}")
    # top-p on the GPU's own scores must match the oracle's rule exactly
    gs = np64(bufs.scores)
    for b in range(B):
        assert_topp_unit(sets[b], gs[b], pf, wl.K_min, wl.K_max, wl.n_sink, wl.n_rec,
                         tag=f"{tag} unit row {b}")
    log(f"{tag}: scores and selection match")
    heads = None
    if check_rows is not None:
        heads = set(check_rows)
    Kr = np64(inp_dev["K"]) if heads is None else _lazy_kv(inp_dev["K"])
    Vr = np64(inp_dev["V"]) if heads is None else _lazy_kv(inp_dev["V"])
    ref = O.sparse_attention(np64(inp_dev["q"]), Kr, Vr, sets, wl.block,
                             1.0 / math.sqrt(wl.d), heads=heads)
    got = np64(bufs.out)
    scale = 1.0 / math.sqrt(wl.d)
    rows = sorted(heads) if heads is not None else \
        [(b, h) for b in range(B) for h in range(wl.Hq)]
    mag = attention_magnitude(inp_dev["q"].float(), inp_dev["K"], inp_dev["V"], sets, wl.block,
                              scale, rows) if dt == torch.bfloat16 else None
    for (b, h) in rows:
        assert_out_close(got[b, h][None], ref[b, h][None], dt, tag=f"{tag} ({b},{h})",
                         mag=None if mag is None else [mag[(b, h)]])
    log(f"{tag}: outputs match")
    return bufs, sets


def _every_kv_head(wl, B=None):
    """One query head of every KV head group of every query (a different one of the
    group from query to query), and the first and last heads."""
    B = wl.B if B is None else B
    rows = {(b, g * wl.G + (b + g) % wl.G) for b in range(B) for g in range(wl.Hkv)}
    return sorted(rows | {(0, 0), (B - 1, wl.Hq - 1)})


class _lazy_kv:
    """Indexable view of a device KV cache that copies one [L][d] slice at a time."""

    def __init__(self, t):
        self.t = t
        self.shape = t.shape

    def __getitem__(self, key):
        b, g = key
        return self.t[b, g].to("cpu", torch.float64).numpy()


@pytest.mark.parametrize("name", ["c1_small_f32", "c2_32k_b4"])
def test_workload_end_to_end(name):
    wl = W.WORKLOADS[name]
    log(f"e2e {name}")
    inp = W.make_inputs(wl, device="cpu")
    dev = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    bufs, sets = run_e2e(wl, dev, tag=name)
    if wl.structure == "planted":
        for b, s in enumerate(sets):
            assert set(inp["planted"][b]) <= set(s), "planted blocks must be selected"
            if name == "c1_small_f32":
                assert len(s) == 7       # 4 tied planted blocks + 3 reserved
            else:
                assert len(s) == 16      # the K_min floor binds


@pytest.fixture(scope="module")
def big_inputs():
    cache = {}

    def get(name):
        if name not in cache:
            cache.clear()
            torch.cuda.empty_cache()
            wl = W.WORKLOADS[name]
            log(f"generating {name} on the GPU")
            cache[name] = W.make_inputs(wl, device=DEV)
            torch.cuda.synchronize()
        return cache[name]
    return get


@pytest.mark.parametrize("name", ["c3_128k_b1", "c3_128k_b8", "c4_128k_b8_int4"])
def test_workload_full_size(name, big_inputs):
    wl = W.WORKLOADS[name]
    inp = big_inputs(name)
    bufs, sets = run_e2e(wl, inp, check_rows=_every_kv_head(wl), tag=name)
    for s in sets:
        if wl.sel_k_dtype == "int4":
            # 4-bit keys add score noise that sharpens the distribution: the nucleus
            # is no longer capped, so only the bounds on |S| hold
            assert wl.K_min <= len(s) <= wl.K_max
        else:
            assert len(s) == wl.K_max     # the Zipf(1.1) nucleus is far above the cap


def test_workload_static_topk_half(big_inputs):
    """Static top-K at half the context (Eq. 6; the paper's K = 0.5L decode rows) on the
    128K batch-8 inputs: 1024 of 2048 blocks per query, sampled outputs."""
    base = W.WORKLOADS["c3_128k_b8"]
    inp = big_inputs(base.name)
    wl = base.with_(p=0.0, K_min=base.nb // 2, K_max=base.nb // 2, n_sink=0, n_rec=0)
    bufs, sets = run_e2e(wl, inp, check_rows=_every_kv_head(wl), tag="c3-static-half")
    assert all(len(s) == wl.nb // 2 for s in sets)


def test_workload_page_geometry(big_inputs):
    """The paper's own geometry end to end at 128K: 16-token blocks, 16 per-token
    selector keys per block (4 heads x 128), Table 3's sink / recency / K_min, p = 0.9
    with no cap. Every score and the whole selection against the oracle, sampled heads
    of the output."""
    wl = W.WORKLOADS["page_128k_b1"]
    inp = big_inputs(wl.name)
    bufs, sets = run_e2e(wl, inp, check_rows=_every_kv_head(wl), tag=wl.name)
    n = len(sets[0])
    assert wl.K_min <= n < wl.nb // 2, n


@pytest.mark.parametrize("kf,qf", [("int8", None), ("fp8", "fp8"), ("fp4", None),
                                   ("fp4", "fp4"), ("int4", "int4")])
def test_workload_selector_formats(kf, qf):
    """The 128K layer (batch 2) with the selector key cache, and optionally the selector
    query, stored in the other precisions of §5.3 / Table 9: all scores, the selection
    and sampled outputs against the oracle on the same codes."""
    wl = W.WORKLOADS["c3_128k_b8"].with_(B=2, sel_k_dtype=kf, sel_q_dtype=qf,
                                         name=f"c3_128k_b2_{kf}_{qf}")
    inp = W.make_inputs(wl, device=DEV)
    bufs, sets = run_e2e(wl, inp, check_rows=_every_kv_head(wl), tag=wl.name)
    assert all(wl.K_min <= len(s) <= wl.K_max for s in sets)


def test_workload_budgets_vary(big_inputs):
    """Zipf exponents spread over [1.3, 2.0] across the batch give different budgets."""
    wl = W.WORKLOADS["c3_128k_b8"].with_(zipf_spread=(1.3, 2.0), L=32768)
    inp = W.make_inputs(wl, device=DEV)
    bufs, sets = run_e2e(wl, inp, check_rows=_every_kv_head(wl), tag="c3-spread")
    sizes = [len(s) for s in sets]
    assert len(set(sizes)) >= 4, sizes


def test_decode_step_bit_reproducible():
    wl = W.WORKLOADS["c2_32k_b4"]
    inp = W.make_inputs(wl, device=DEV, seed=7)
    outs = []
    for _ in range(2):
        bufs = DecodeBuffers.of(wl, torch.bfloat16)
        decode_step(inp, wl, bufs)
        outs.append((bufs.scores.cpu(), bufs.sel_idx.cpu(), bufs.out.cpu()))
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b)


def test_prepared_step_matches_decode_step():
    """The decode step with its calls marshalled once (DecodeStep, what the benchmark
    times) writes exactly what decode_step writes, call after call."""
    wl = W.WORKLOADS["c2_32k_b4"]
    inp = W.make_inputs(wl, device=DEV, seed=13)
    ref = DecodeBuffers.of(wl, torch.bfloat16)
    decode_step(inp, wl, ref)
    bufs = DecodeBuffers.of(wl, torch.bfloat16)
    stream = torch.cuda.Stream()
    step = DecodeStep(inp, wl, bufs, stream=stream)
    torch.cuda.synchronize()
    for _ in range(3):
        bufs.out.fill_(float("nan"))
        bufs.sel_idx.fill_(-5)
        torch.cuda.synchronize()
        step()
        torch.cuda.synchronize()
        for name in ("scores", "sel_idx", "sel_cnt", "sel_mass", "out"):
            assert torch.equal(getattr(bufs, name), getattr(ref, name)), name


def test_graph_replay_matches_eager():
    """The decode step captured in a HIP graph: every replay, with eager work and
    synchronisations in between, reproduces the eager result bit for bit."""
    wl = W.WORKLOADS["c2_32k_b4"]
    inp = W.make_inputs(wl, device=DEV, seed=11)
    eager = DecodeBuffers.of(wl, torch.bfloat16)
    decode_step(inp, wl, eager)
    torch.cuda.synchronize()
    ref = (eager.sel_idx.clone(), eager.sel_cnt.clone(), eager.out.clone())
    bufs = DecodeBuffers.of(wl, torch.bfloat16)
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        decode_step(inp, wl, bufs, stream=stream)
    for i in range(4):
        bufs.out.fill_(float("nan"))
        bufs.sel_idx.fill_(12345)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        decode_step(inp, wl, eager)           # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(bufs.sel_idx, ref[0]) and torch.equal(bufs.sel_cnt, ref[1])
        assert torch.equal(bufs.out, ref[2]), f"replay {i}"


@pytest.mark.parametrize("spread", [None, (1.3, 2.0)], ids=["equal_budgets", "spread_budgets"])
def test_graph_replay_headline_shape_dirty_workspace(spread):
    """The 128K batch-8 decode step (runs cut across the batch, the merge stopping at each
    query's flagged last slot) captured in a HIP graph as a server would: every replay,
    with the workspace overwritten by 0xFF bytes (NaN partials) and the outputs poisoned
    between replays, reproduces the stream-launched step bit for bit. With budgets spread
    over the batch (Zipf 1.3-2.0 per row) the runs span two or three queries each."""
    wl = W.WORKLOADS["c3_128k_b8"]
    if spread is not None:
        wl = wl.with_(zipf_spread=spread)
    log(f"graph replay c3_128k_b8 spread={spread}")
    inp = W.make_inputs(wl, device=DEV)
    bufs = DecodeBuffers.of(wl, inp["q"].dtype)
    stream = torch.cuda.Stream()
    step = DecodeStep(inp, wl, bufs, stream=stream)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        step()
    torch.cuda.synchronize()
    ref = (bufs.scores.clone(), bufs.sel_idx.clone(), bufs.sel_cnt.clone(), bufs.out.clone())
    if spread is not None:  # the rows really select different numbers of blocks
        assert len(set(bufs.sel_cnt.tolist())) > 2, bufs.sel_cnt.tolist()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        step()
    for i in range(3):
        bufs.workspace.fill_(255)
        bufs.out.fill_(float("nan"))
        bufs.sel_idx.fill_(-3)
        bufs.scores.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, r in zip(("scores", "sel_idx", "sel_cnt", "out"), ref):
            assert torch.equal(getattr(bufs, name), r), f"replay {i}: {name}"
    del g


def test_page_geometry_scoring_sampled():
    """The paper's selector geometry (per-token keys, 16 per block, 4 heads x 128) at a
    128K context, batch 1: sampled blocks against the oracle, then the top-p rule on the
    GPU's own scores."""
    nb, kpb, H, di = 8192, 16, 4, 128
    g = torch.Generator(device=DEV)
    g.manual_seed(3)
    sel_q = torch.randn(1, H, di, generator=g, device=DEV).bfloat16()
    sel_w = torch.randn(1, H, generator=g, device=DEV).abs()
    sel_k = torch.randn(1, nb, kpb, H, di, generator=g, device=DEV).bfloat16()
    scores = torch.empty(1, nb, device=DEV)
    _lib.spot_select_score(sel_q, sel_w, sel_k, None, scores, kpb=kpb)
    idx = torch.empty(1, nb, dtype=torch.int32, device=DEV)
    cnt = torch.empty(1, dtype=torch.int32, device=DEV)
    _lib.spot_select_topp(scores, idx, cnt, None, 0.9, 32, nb, 8, 16)
    torch.cuda.synchronize()
    pick = torch.tensor([0, 1, 2, 777, 4096, 8190, 8191] + list(range(3000, 3064)))
    keys = np64(sel_k[:, pick])
    ref = O.select_score(np64(sel_q), np64(sel_w), keys)
    assert_scores_close(np64(scores)[:, pick.numpy()], ref,
                        score_magnitude(np64(sel_q), np64(sel_w), keys))
    s = gpu_sets(idx, cnt)[0]
    assert_topp_unit(s, np64(scores)[0], float(np.float32(0.9)), 32, nb, 8, 16, tag="page")
