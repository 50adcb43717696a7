"""GPU parity of the prefill-tile variant: MFMA tile scoring, top-p over the visible
blocks with the diagonal recency window, and causal block-sparse MFMA attention."""
import math

import numpy as np
import pytest
import torch

from block_sparse_long_spot_amd import _lib
from block_sparse_long_spot_amd import workloads as W
from oracle import spot_oracle as O
from parity import (assert_out_close, assert_scores_close, assert_selection_e2e,
                    assert_topp_unit, decode_selector, gpu_sets, np64, tile_score_magnitude)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def log(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    _lib.load()


SCORE_CASES = [
    # B, Tq, q_pos0, nb_cache, kpb, H, d_idx
    (1, 128, 32640, 512, 1, 4, 64),
    (2, 40, 1000, 20, 1, 4, 64),
    (1, 17, 0, 1, 2, 2, 32),
    (1, 128, 200, 6, 1, 1, 128),
    (2, 100, 5000, 100, 3, 4, 64),
    (1, 64, 4095, 70, 1, 8, 32),
]


@pytest.mark.parametrize("case", SCORE_CASES, ids=lambda c: "-".join(map(str, c)))
def test_prefill_score_parity(case):
    B, Tq, q_pos0, nb_cache, kpb, H, di = case
    log(f"prefill score {case}")
    g = torch.Generator().manual_seed(Tq + q_pos0)
    sel_q = torch.randn(B, Tq, H, di, generator=g).bfloat16()
    sel_w = torch.randn(B, Tq, H, generator=g)
    sel_k = torch.randn(B, nb_cache, kpb, H, di, generator=g).bfloat16()
    nb_vis = -(-(q_pos0 + Tq) // 64)
    scores = torch.full((B, nb_vis), float("nan"), device=DEV)
    _lib.spot_prefill_select_score(sel_q.to(DEV), sel_w.to(DEV), sel_k.to(DEV), scores, q_pos0,
                                   block=64, kpb=kpb)
    torch.cuda.synchronize()
    ref = O.prefill_tile_score(np64(sel_q), np64(sel_w), np64(sel_k), q_pos0, 64)
    mag = tile_score_magnitude(np64(sel_q), np64(sel_w), np64(sel_k), q_pos0, 64)
    assert_scores_close(np64(scores), ref, mag)


QUANT_SCORE_CASES = [
    # key format, B, T, Tq, q_pos0, nb_cache, kpb, H, d_idx (T == Tq: one tile)
    ("int4", 1, 128, 128, 32640, 512, 1, 4, 64),
    ("fp4", 1, 128, 128, 32640, 512, 1, 4, 64),
    ("int8", 2, 40, 40, 1000, 20, 1, 4, 64),
    ("fp8", 2, 40, 40, 1000, 20, 2, 4, 128),
    ("int4", 1, 100, 100, 5000, 100, 3, 4, 32),
    ("fp4", 1, 64, 64, 4095, 70, 1, 8, 32),          # any-H path
    ("int4", 1, 17, 17, 0, 1, 2, 2, 128),             # any-H path, one block
    # a whole sequence in tiles (>= 2048 tile x column-group pairs: many groups per
    # work-group)
    ("int4", 1, 8192, 128, 24576, 512, 1, 4, 64),
    ("fp4", 1, 8192, 128, 24576, 512, 1, 4, 64),
    ("fp8", 2, 4000, 100, 28000, 500, 1, 4, 64),
]


@pytest.mark.parametrize("case", QUANT_SCORE_CASES, ids=lambda c: "-".join(map(str, c)))
def test_prefill_score_quantised_keys(case):
    """Tile scores with the selector key cache in the quantised formats of §5.3, against
    the oracle's tile scores on the same codes decoded (a bf16 query)."""
    fmt, B, T, Tq, q_pos0, nb_cache, kpb, H, di = case
    log(f"prefill score quantised {case}")
    if T > Tq:   # the launch takes the path with many column groups per work-group
        assert B * (-(-T // Tq)) * -(-(-(-(q_pos0 + T) // 64)) // 16) >= 2048
    g = torch.Generator().manual_seed(T + q_pos0 + di)
    sel_q = torch.randn(B, T, H, di, generator=g).bfloat16()
    sel_w = torch.randn(B, T, H, generator=g)                 # signed weights
    codes, kscale = W.quantize_selector(torch.randn(B, nb_cache, kpb, H, di, generator=g), fmt)
    n_tiles = -(-T // Tq)
    nb_seq = -(-(q_pos0 + T) // 64)
    scores = torch.full((B, n_tiles, nb_seq), float("nan"), device=DEV)
    _lib.spot_prefill_select_score(sel_q.to(DEV), sel_w.to(DEV), codes.to(DEV), scores, q_pos0,
                                   block=64, kpb=kpb, Tq=Tq, sel_k_scale=kscale.to(DEV))
    torch.cuda.synchronize()
    keys = decode_selector(codes, kscale)
    sq, sw, gs = np64(sel_q), np64(sel_w), np64(scores)
    for t in sorted({0, n_tiles // 2, n_tiles - 1}):
        q0, q1 = t * Tq, min((t + 1) * Tq, T)
        nb_t = -(-(q_pos0 + q1) // 64)
        ref = O.prefill_tile_score(sq[:, q0:q1], sw[:, q0:q1], keys, q_pos0 + q0, 64)
        assert_scores_close(gs[:, t, :nb_t], ref,
                            tile_score_magnitude(sq[:, q0:q1], sw[:, q0:q1], keys, q_pos0 + q0,
                                                 64))


SEQ_SCORE_CASES = [
    # B, T, Tq, q_pos0, block, kpb, d_idx, weights at a 4-byte (not 16-byte) address,
    # tiles checked. Each launch has >= 2048 (tile, 16-block column group) pairs, so a
    # work-group scores several column groups with one load of its tile's queries.
    (1, 1024, 16, 7168, 16, 2, 32, True, (0, 1, 31, 63)),
    (2, 2000, 100, 30000, 32, 1, 64, False, (0, 7, 19)),
    (1, 4000, 128, 62000, 64, 1, 128, True, (0, 13, 31)),
]


@pytest.mark.parametrize("case", SEQ_SCORE_CASES, ids=lambda c: "-".join(map(str, c[:8])))
def test_prefill_sequence_score_parity(case):
    B, T, Tq, q_pos0, block, kpb, di, unaligned, tiles = case
    log(f"prefill sequence score {case}")
    H = 4
    nb_seq = -(-(q_pos0 + T) // block)
    n_tiles = -(-T // Tq)
    assert B * n_tiles * -(-nb_seq // 16) >= 2048
    g = torch.Generator().manual_seed(T + q_pos0)
    sel_q = torch.randn(B, T, H, di, generator=g).bfloat16()
    w = torch.rand(B * T * H + 1, generator=g)
    sel_k = torch.randn(B, nb_seq, kpb, H, di, generator=g).bfloat16()
    wd = w.to(DEV)
    sel_w = (wd[1:] if unaligned else wd[:-1]).view(B, T, H)
    assert (sel_w.data_ptr() % 16 != 0) == unaligned
    scores = torch.full((B, n_tiles, nb_seq), float("nan"), device=DEV)
    _lib.spot_prefill_select_score(sel_q.to(DEV), sel_w, sel_k.to(DEV), scores, q_pos0,
                                   block=block, kpb=kpb, Tq=Tq)
    torch.cuda.synchronize()
    sq, sw, sk, gs = np64(sel_q), np64(sel_w.cpu()), np64(sel_k), np64(scores)
    for t in tiles:
        q0, q1 = t * Tq, min((t + 1) * Tq, T)
        nb_t = -(-(q_pos0 + q1) // block)
        ref = O.prefill_tile_score(sq[:, q0:q1], sw[:, q0:q1], sk, q_pos0 + q0, block)
        assert_scores_close(gs[:, t, :nb_t], ref,
                            tile_score_magnitude(sq[:, q0:q1], sw[:, q0:q1], sk, q_pos0 + q0,
                                                 block))
        assert np.isnan(gs[:, t, nb_t:]).all()  # blocks after the tile are not written


ATTN_CASES = [
    # B, Hq, Hkv, Tq, q_pos0, L, pattern
    (1, 32, 8, 128, 32640, 32768, "random"),
    (1, 8, 2, 128, 1000, 1128, "all"),
    (2, 8, 8, 40, 300, 400, "random"),
    (1, 4, 2, 17, 0, 17, "all"),
    (1, 16, 2, 100, 5000, 7000, "with_future"),
    (2, 8, 1, 64, 64, 1000, "random"),
    (1, 8, 4, 128, 700, 900, "diag_only"),
    (1, 8, 2, 33, 2000, 2100, "empty"),
    (1, 8, 1, 16, 524272, 524288, "all"),     # the longest list: 8192 selected blocks
]


def _prefill_sets(pattern, B, q_pos0, Tq, L, g):
    nb = -(-L // 64)
    last = (q_pos0 + Tq - 1) // 64
    sets = []
    for b in range(B):
        if pattern == "all":
            s = list(range(last + 1))
        elif pattern == "diag_only":
            s = list(range(max(0, last - 3), last + 1))
        elif pattern == "empty":
            s = []
        else:
            pool = torch.randperm(last + 1, generator=g)[: max(1, (last + 1) // 3)].tolist()
            s = set(pool) | set(range(max(0, last - 3), last + 1)) | {0}
            if pattern == "with_future" and last + 1 < nb:
                s |= {last + 1, nb - 1}       # blocks after the tile: fully masked
            s = sorted(s)
        sets.append(s)
    return sets


@pytest.mark.parametrize("case", ATTN_CASES, ids=lambda c: "-".join(map(str, c)))
def test_prefill_attn_parity(case):
    B, Hq, Hkv, Tq, q_pos0, L, pattern = case
    log(f"prefill attn {case}")
    g = torch.Generator().manual_seed(L + Tq)
    Q = torch.randn(B, Hq, Tq, 128, generator=g).bfloat16()
    K = torch.randn(B, Hkv, L, 128, generator=g).bfloat16()
    V = torch.randn(B, Hkv, L, 128, generator=g).bfloat16()
    sets = _prefill_sets(pattern, B, q_pos0, Tq, L, g)
    K_max = max(1, max(len(s) for s in sets))
    idx = torch.full((B, K_max), -1, dtype=torch.int32)
    cnt = torch.zeros(B, dtype=torch.int32)
    for b, s in enumerate(sets):
        if s:
            idx[b, : len(s)] = torch.tensor(s, dtype=torch.int32)
        cnt[b] = len(s)
    out = torch.full((B, Hq, Tq, 128), float("nan"), device=DEV).bfloat16()
    scale = 1 / math.sqrt(128)
    _lib.spot_prefill_attn(Q.to(DEV), K.to(DEV), V.to(DEV), idx.to(DEV), cnt.to(DEV), out, q_pos0,
                           scale)
    torch.cuda.synchronize()
    ref = O.prefill_attention(np64(Q), np64(K), np64(V), sets, 64, scale, q_pos0)
    assert_out_close(np64(out), ref, torch.bfloat16, tag=str(case))


@pytest.mark.parametrize("scale", [-1 / math.sqrt(128), 0.0, 0.5])
def test_prefill_attn_scale_sign_and_zero(scale):
    """The softmax scale is folded into the exponential: a negative scale (the kernel
    negates q instead), a zero scale (uniform weights over the visible tokens) and a
    large one, on a diagonal tile with a ragged end."""
    B, Hq, Hkv, Tq, q_pos0, L = 1, 8, 2, 40, 300, 340
    log(f"prefill attn scale {scale}")
    g = torch.Generator().manual_seed(77)
    Q = torch.randn(B, Hq, Tq, 128, generator=g).bfloat16()
    K = torch.randn(B, Hkv, L, 128, generator=g).bfloat16()
    V = torch.randn(B, Hkv, L, 128, generator=g).bfloat16()
    sets = [[0, 2, 4, 5]]
    idx = torch.tensor([sets[0]], dtype=torch.int32)
    cnt = torch.tensor([4], dtype=torch.int32)
    out = torch.full((B, Hq, Tq, 128), float("nan"), device=DEV).bfloat16()
    _lib.spot_prefill_attn(Q.to(DEV), K.to(DEV), V.to(DEV), idx.to(DEV), cnt.to(DEV), out, q_pos0,
                           scale)
    torch.cuda.synchronize()
    ref = O.prefill_attention(np64(Q), np64(K), np64(V), sets, 64, scale, q_pos0)
    assert_out_close(np64(out), ref, torch.bfloat16, tag=f"scale {scale}")


def test_prefill_tile_end_to_end():
    """The 128-query tile at positions 32640..32767 of a 32K context."""
    wl = W.WORKLOADS["c5_prefill_32k"]
    inp = W.make_inputs(wl, device=DEV)
    q_pos0, Tq, nb_vis = wl.q_pos0, wl.prefill_Tq, wl.nb
    scores = torch.empty(wl.B, nb_vis, device=DEV)
    _lib.spot_prefill_select_score(inp["sel_q"], inp["sel_w"], inp["sel_k"], scores, q_pos0)
    K_max = nb_vis
    idx = torch.empty(wl.B, K_max, dtype=torch.int32, device=DEV)
    cnt = torch.empty(wl.B, dtype=torch.int32, device=DEV)
    _lib.spot_select_topp(scores, idx, cnt, None, wl.p, wl.K_min, K_max, wl.n_sink, wl.n_rec)
    out = torch.empty(wl.B, wl.Hq, Tq, wl.d, dtype=torch.bfloat16, device=DEV)
    scale = 1 / math.sqrt(wl.d)
    _lib.spot_prefill_attn(inp["q"], inp["K"], inp["V"], idx, cnt, out, q_pos0, scale)
    torch.cuda.synchronize()
    sq, sw, sk = np64(inp["sel_q"]), np64(inp["sel_w"]), np64(inp["sel_k"])
    ref_s = O.prefill_tile_score(sq, sw, sk, q_pos0, wl.block)
    assert_scores_close(np64(scores), ref_s, tile_score_magnitude(sq, sw, sk, q_pos0, wl.block))
    sets = gpu_sets(idx, cnt)
    pf = float(np.float32(wl.p))
    assert_selection_e2e(sets[0], ref_s[0], pf, wl.K_min, K_max, wl.n_sink, wl.n_rec, "c5")
    assert_topp_unit(sets[0], np64(scores)[0], pf, wl.K_min, K_max, wl.n_sink, wl.n_rec, "c5u")
    assert set(range(nb_vis - 4, nb_vis)) <= set(sets[0]) and 0 in sets[0]
    log(f"c5: |S| = {len(sets[0])} of {nb_vis} blocks")
    heads = {(0, h) for h in (0, 5, 17, 31)}
    ref = O.prefill_attention(np64(inp["q"]), _KV(inp["K"]), _KV(inp["V"]), sets, wl.block,
                              scale, q_pos0, heads=heads)
    got = np64(out)
    for (b, h) in heads:
        assert_out_close(got[b, h], ref[b, h], torch.bfloat16, tag=f"c5 head {h}")


class _KV:
    def __init__(self, t):
        self.t, self.shape = t, t.shape

    def __getitem__(self, key):
        b, g = key
        return self.t[b, g].to("cpu", torch.float64).numpy()


def _sequence_case(B, T, Tq, q_pos0, Hq, Hkv, p, n_sink, n_rec, K_min, seed, tiles_checked,
                   heads_checked, K_max=None):
    """Whole-sequence prefill through the three tile-indexed calls, checked per tile
    against the oracle: every score of the checked tiles, their selection (on the GPU's
    own scores and end to end) and the outputs of the checked heads."""
    d, H, di, block = 128, 4, 64, 64
    L = q_pos0 + T
    nb_seq = -(-L // block)
    n_tiles = -(-T // Tq)
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    sel_q = torch.randn(B, T, H, di, generator=g, device=DEV).bfloat16()
    sel_w = torch.rand(B, T, H, generator=g, device=DEV)
    sel_k = torch.randn(B, nb_seq, 1, H, di, generator=g, device=DEV).bfloat16()
    Q = torch.randn(B, Hq, T, d, generator=g, device=DEV).bfloat16()
    K = torch.randn(B, Hkv, L, d, generator=g, device=DEV).bfloat16()
    V = torch.randn(B, Hkv, L, d, generator=g, device=DEV).bfloat16()
    scores = torch.full((B, n_tiles, nb_seq), float("nan"), device=DEV)
    _lib.spot_prefill_select_score(sel_q, sel_w, sel_k, scores, q_pos0, Tq=Tq)
    K_max = nb_seq if K_max is None else K_max
    idx = torch.full((B, n_tiles, K_max), 12345, dtype=torch.int32, device=DEV)
    cnt = torch.full((B, n_tiles), -1, dtype=torch.int32, device=DEV)
    _lib.spot_prefill_select_topp(scores, idx, cnt, None, p, K_min, K_max, n_sink, n_rec,
                                  q_pos0, T, Tq=Tq)
    out = torch.full((B, Hq, T, d), float("nan"), device=DEV).bfloat16()
    scale = 1 / math.sqrt(d)
    _lib.spot_prefill_attn(Q, K, V, idx, cnt, out, q_pos0, scale, Tq=Tq)
    torch.cuda.synchronize()
    log(f"sequence B{B} T{T} Tq{Tq} q_pos0 {q_pos0}: {n_tiles} tiles on the GPU")
    sq, sw, sk = np64(sel_q), np64(sel_w), np64(sel_k)
    gs, got = np64(scores), np64(out)
    pf = float(np.float32(p))
    sizes = []
    for t in tiles_checked:
        q0, q1 = t * Tq, min((t + 1) * Tq, T)
        nb_t = -(-(q_pos0 + q1) // block)
        ref_s = O.prefill_tile_score(sq[:, q0:q1], sw[:, q0:q1], sk, q_pos0 + q0, block)
        assert ref_s.shape[1] == nb_t
        assert_scores_close(gs[:, t, :nb_t], ref_s,
                            tile_score_magnitude(sq[:, q0:q1], sw[:, q0:q1], sk, q_pos0 + q0,
                                                 block))
        sets = gpu_sets(idx[:, t], cnt[:, t])
        for b in range(B):
            assert_topp_unit(sets[b], gs[b, t, :nb_t], pf, K_min, K_max, n_sink, n_rec,
                             tag=f"tile {t} row {b}")
            assert_selection_e2e(sets[b], ref_s[b], pf, K_min, K_max, n_sink, n_rec,
                                 tag=f"tile {t} e2e {b}")
            assert max(sets[b]) < nb_t and set(range(max(nb_t - n_rec, 0), nb_t)) <= set(sets[b])
            sizes.append(len(sets[b]))
        heads = {(b, h) for b in range(B) for h in heads_checked}
        ref = O.prefill_attention(np64(Q[:, :, q0:q1]), _KV(K), _KV(V), sets, block, scale,
                                  q_pos0 + q0, heads=heads)
        for (b, h) in heads:
            assert_out_close(got[b, h, q0:q1], ref[b, h], torch.bfloat16, tag=f"tile {t} ({b},{h})")
    log(f"checked tiles {list(tiles_checked)}: |S| {sizes}")


def test_prefill_sequence_ragged():
    """1000 queries from position 48 in tiles of 128 (the last has 104): every tile."""
    _sequence_case(B=2, T=1000, Tq=128, q_pos0=48, Hq=8, Hkv=2, p=0.9, n_sink=1, n_rec=4,
                   K_min=0, seed=31, tiles_checked=range(8), heads_checked=range(8))


def test_prefill_sequence_two_heads_per_wave_ragged():
    """Grids large enough for two heads per wave: 100-query tiles (7 row tiles, so the
    last pair has one idle wave) with a 50-query last tile, and 128-query tiles with a
    32-query last tile; both heads of each wave's pair are checked."""
    _sequence_case(B=2, T=1450, Tq=100, q_pos0=37, Hq=32, Hkv=8, p=0.9, n_sink=1, n_rec=4,
                   K_min=0, seed=33, tiles_checked=(0, 7, 14), heads_checked=(0, 1, 2, 3, 31))
    _sequence_case(B=1, T=4000, Tq=128, q_pos0=100, Hq=32, Hkv=8, p=0.95, n_sink=1, n_rec=4,
                   K_min=8, seed=34, tiles_checked=(0, 16, 31), heads_checked=(0, 1, 6, 7, 30))


def test_prefill_edge_lists_large_grid():
    """Hand-made lists on a two-heads-per-wave grid of 4096 work-groups (128 tiles of 128
    x 8 KV heads), from position 10 so that 32-row work-groups and 64-token blocks do not
    align, with L ending inside the last block: an empty list (every row zero); a list
    whose only block starts after the first 32 rows' last query (those rows are zero, the
    next 32 attend); invalid, future and unsorted entries; a 130-block list. Every
    checked row is compared, so rows left unwritten (NaN) fail."""
    B, Hq, Hkv, Tq, q_pos0, T, K_max = 1, 32, 8, 128, 10, 128 * 128, 160
    L = q_pos0 + T
    nb = -(-L // 64)
    n_tiles = T // Tq
    log(f"prefill edge lists, {n_tiles} tiles")
    g = torch.Generator(device=DEV)
    g.manual_seed(39)
    Q = torch.randn(B, Hq, T, 128, generator=g, device=DEV).bfloat16()
    K = torch.randn(B, Hkv, L, 128, generator=g, device=DEV).bfloat16()
    V = torch.randn(B, Hkv, L, 128, generator=g, device=DEV).bfloat16()
    lists = {}
    for t in range(n_tiles):
        diag = (q_pos0 + t * Tq + Tq - 1) // 64
        lists[t] = [0, diag]
    lists[0] = []
    lists[1] = [3]                         # first token 192: rows 0-31 (138..169) see none
    lists[2] = [-1, 0, 300, 200, 4, 2]     # invalid, beyond nb, future, then visible ones
    lists[64] = list(range(130))
    lists[127] = [nb - 1, nb - 3, 0]       # the block crossing L first, unsorted
    idx = torch.full((B, n_tiles, K_max), -1, dtype=torch.int32)
    cnt = torch.zeros(B, n_tiles, dtype=torch.int32)
    for t, lst in lists.items():
        if lst:
            idx[0, t, : len(lst)] = torch.tensor(lst, dtype=torch.int32)
        cnt[0, t] = len(lst)
    out = torch.full((B, Hq, T, 128), float("nan"), device=DEV).bfloat16()
    scale = 1 / math.sqrt(128)
    _lib.spot_prefill_attn(Q, K, V, idx.to(DEV), cnt.to(DEV), out, q_pos0, scale, Tq=Tq)
    torch.cuda.synchronize()
    heads = {(0, h) for h in (0, 1, 2, 3, 17, 31)}
    got = np64(out)
    for t in (0, 1, 2, 64, 127):
        q0, q1 = t * Tq, (t + 1) * Tq
        sets = [sorted(b for b in lists[t] if 0 <= b < nb)]
        ref = O.prefill_attention(np64(Q[:, :, q0:q1]), _KV(K), _KV(V), sets, 64, scale,
                                  q_pos0 + q0, heads=heads)
        for (b, h) in heads:
            assert_out_close(got[b, h, q0:q1], ref[b, h], torch.bfloat16, tag=f"tile {t} head {h}")
    assert not np.isnan(got[0, :, : 2 * Tq]).any()
    assert (got[0, :, :Tq] == 0).all() and (got[0, :, Tq : Tq + 32] == 0).all()


def test_prefill_sequence_long_list_stride():
    """A list stride of 8192 entries (the longest list) on a grid of 1024 row tiles: the
    list takes 32 KiB of LDS beside the two 32 KiB block buffers, so one work-group fits
    per CU instead of two."""
    _sequence_case(B=1, T=2048, Tq=128, q_pos0=0, Hq=32, Hkv=8, p=0.95, n_sink=1, n_rec=4,
                   K_min=2, seed=36, tiles_checked=(0, 9, 15), heads_checked=(0, 3, 29),
                   K_max=8192)


def test_prefill_sequence_mid_grid():
    """512 one-head work-groups (between the split-list and two-heads-per-wave forms)."""
    _sequence_case(B=1, T=1000, Tq=128, q_pos0=0, Hq=32, Hkv=8, p=0.9, n_sink=1, n_rec=4,
                   K_min=4, seed=35, tiles_checked=(0, 3, 7), heads_checked=(0, 5, 31))


def test_prefill_sequence_32k():
    """A whole 32K prefill (256 tiles of 128, the c5 layer shape), sampled tiles."""
    _sequence_case(B=1, T=32768, Tq=128, q_pos0=0, Hq=32, Hkv=8, p=0.95, n_sink=1, n_rec=4,
                   K_min=0, seed=32, tiles_checked=(0, 1, 2, 37, 128, 200, 255),
                   heads_checked=(0, 13, 31))
