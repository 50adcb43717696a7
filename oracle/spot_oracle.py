"""CPU oracle for the SpotAttention decode and prefill hot path.

TEST INFRASTRUCTURE ONLY. Nothing but the tests, the smoke check and the
benchmark's CPU-baseline leg may import or call this module; the product path
never does. It shares no code with the HIP library and imports nothing from it.

Plain, slow and obviously correct: every quantity is widened to float64 and each
step follows the paper's definitions in the paper's order, with library
primitives (einsum, sort, cumsum, exp) as the only building blocks and no
blocking, fusion or reordering of the arithmetic.

Source: "SpotAttention: Plug-In Block-Sparse Routing for Pretrained Long-Context
Transformers" (Ahmad and Yun). Sections cited below are that paper's.

Readings where the paper is silent or open (each is listed with its reason in the
design notes of the repository):
  * scores carry no 1/sqrt(d_idx) factor and the softmax temperature is 1 (§2.1 gives
    the bare formula; Appendix A, Table 3 lists temperature 1.0);
  * K_min and K_max bound the total set size |S_q| (Eq. 8 states the floor on |S_q|;
    the cap is the same kind of bound), so the nucleus is clamped to
    [K_min - r, K_max - r] where r = |S_sink u S_rec|;
  * "reaches p" means cumulative residual mass >= p; p >= 1 keeps every residual
    block, p <= 0 keeps none before the floor;
  * ties in score are broken by the lower block index; -0.0 equals +0.0;
  * an empty selected set gives a zero output row;
  * the selected set is reported in ascending block order.

Every function here is pinned by tests/test_oracle_pins.py to closed forms,
brute force on tiny inputs, textbook library routines or figures printed in the
paper; no function is "parity unpinned".
"""
from __future__ import annotations

import numpy as np


# ---------------------------------------------------------------------------
# Selector K-cache decoding (§5.3 and Appendix G: INT4 microscale, group 32,
# 4.5 bits per element = 4-bit codes plus one 16-bit scale per 32 elements).
# ---------------------------------------------------------------------------
def dequant_int4_g32(codes, scales):
    """Decode INT4 codes with one fp16 scale per 32 elements.

    codes  uint8 [..., n/2]: element 2i in the low nibble, element 2i+1 in the high
           nibble, each a two's-complement value in [-8, 7];
    scales float16 [..., n/32].
    Returns float64 [..., n] with value = code * scale, computed exactly.
    """
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.float16).astype(np.float64)
    lo = (codes & 0x0F).astype(np.int64)
    hi = (codes >> 4).astype(np.int64)
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    n = codes.shape[-1] * 2
    vals = np.empty(codes.shape[:-1] + (n,), dtype=np.float64)
    vals[..., 0::2] = lo
    vals[..., 1::2] = hi
    scale_per_elem = np.repeat(scales, 32, axis=-1)
    assert scale_per_elem.shape == vals.shape
    return vals * scale_per_elem


# ---------------------------------------------------------------------------
# The other selector-cache precisions of §5.3 and Appendix G (Table 9): INT8 and FP8
# at 0.500x the BF16 footprint (so no per-group scale: one scale for the tensor), and
# FP4 microscale at group 32. The FP4 scale is read as an 8-bit power of two (E8M0):
# §5.3 prints 1.20 GiB for FP4 against 1.27 GiB for INT4 from the same 4.50 GiB, i.e.
# 4.25 bits per element, one byte of scale per 32 elements.
# ---------------------------------------------------------------------------
def dequant_int8(codes, scale):
    """Decode INT8 codes (two's complement) with one scale for the whole tensor:
    value = code * scale, exactly. codes int8 [...]; scale a float32 number."""
    c = np.asarray(codes).astype(np.int8).astype(np.float64)
    return c * float(np.float32(scale))


def decode_fp8_e4m3(codes):
    """FP8 E4M3 (1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; subnormals
    at exponent 0; no infinities; exponent and mantissa all ones is NaN): float64."""
    b = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 0x7).astype(np.float64)
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** (1 - 7), (1.0 + m / 8.0) * 2.0 ** (e - 7.0))
    mag = np.where((e == 15) & (b & 0x7 == 7), np.nan, mag)
    return sign * mag


def dequant_fp8_e4m3(codes, scale):
    """FP8 E4M3 codes times one scale for the whole tensor, exactly."""
    return decode_fp8_e4m3(codes) * float(np.float32(scale))


def decode_fp4_e2m1(nibbles):
    """FP4 E2M1 (1 sign bit, 2 exponent bits with bias 1, 1 mantissa bit; exponent 0
    is subnormal): the 16 codes are +-{0, 0.5, 1, 1.5, 2, 3, 4, 6}. float64."""
    n = np.asarray(nibbles).astype(np.int64) & 0xF
    sign = np.where(n & 0x8, -1.0, 1.0)
    e = (n >> 1) & 0x3
    m = (n & 0x1).astype(np.float64)
    mag = np.where(e == 0, m * 0.5, (1.0 + m / 2.0) * 2.0 ** (e - 1.0))
    return sign * mag


def decode_e8m0(codes):
    """E8M0 scale: 2 ** (code - 127); code 255 is NaN. float64."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.float64)
    return np.where(c == 255, np.nan, 2.0 ** (c - 127.0))


def dequant_fp4_e2m1_g32(codes, scales):
    """FP4 E2M1 codes, two per byte (element 2i in the low nibble), with one E8M0 scale
    byte per 32 elements: value = fp4 * 2 ** (scale - 127), exactly.
    codes uint8 [..., n/2]; scales uint8 [..., n/32]. Returns float64 [..., n]."""
    codes = np.asarray(codes, dtype=np.uint8)
    n = codes.shape[-1] * 2
    vals = np.empty(codes.shape[:-1] + (n,), dtype=np.float64)
    vals[..., 0::2] = decode_fp4_e2m1(codes & 0x0F)
    vals[..., 1::2] = decode_fp4_e2m1(codes >> 4)
    scale_per_elem = np.repeat(decode_e8m0(scales), 32, axis=-1)
    assert scale_per_elem.shape == vals.shape
    return vals * scale_per_elem


# ---------------------------------------------------------------------------
# Quantisation of new selector keys into the cache formats (the write side of
# §5.3: the selector is trained in BF16 and quantised at inference). Where a float
# decides an integer code, the decision is taken in float32, as the kernel takes it:
# the quotient x / scale is a correctly rounded float32 division, then rounded to the
# nearest integer, ties to even.
# ---------------------------------------------------------------------------
def _f32_quotient(x, s):
    return (np.asarray(x, np.float32) / np.float32(s)).astype(np.float32)


def quantize_int4_g32(x):
    """Per group of 32: scale = fp16(amax / 7) (float32 quotient, rounded to fp16 to
    nearest even); code = clamp(rne(x / scale), -8, 7), 0 when the scale is 0; two
    codes per byte, element 2i in the low nibble. x float32 [..., n]. Returns (codes
    uint8 [..., n/2], scales float16 [..., n/32])."""
    x = np.asarray(x, np.float32)
    *lead, n = x.shape
    g = x.reshape(*lead, n // 32, 32)
    amax = np.abs(g).max(axis=-1)
    scale = (amax / np.float32(7)).astype(np.float32).astype(np.float16)
    sf = scale.astype(np.float32)[..., None]
    safe = np.where(sf > 0, sf, np.float32(1))
    q = np.rint(_f32_quotient(g, 1) / safe).astype(np.float32)
    q = np.where(sf > 0, np.clip(q, -8, 7), 0).astype(np.int64).reshape(*lead, n)
    nib = (q & 0xF).astype(np.uint8)
    return (nib[..., 0::2] | (nib[..., 1::2] << 4)), scale


def fp4_group_exponent(amax):
    """The smallest integer e with amax <= 6 * 2^e (exact: from the binary exponent of
    amax), clamped to [-127, 127]; -127 for amax = 0."""
    amax = np.asarray(amax, np.float64)
    m, k = np.frexp(amax)                       # amax = m * 2^k, m in [0.5, 1)
    e = np.where(m <= 0.75, k - 3, k - 2)
    e = np.where(amax > 0, e, -127)
    return np.clip(e, -127, 127).astype(np.int64)


def e2m1_nearest(y):
    """Code (0..7) of the E2M1 magnitude nearest to |y| <= 6, ties to the even code."""
    a = np.abs(np.asarray(y, np.float64))
    mags = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    d = np.abs(a[..., None] - mags)
    best = d.min(axis=-1, keepdims=True)
    cand = d == best                                    # one or two nearest codes
    even = cand & (np.arange(8) % 2 == 0)
    return np.where(even.any(-1), even.argmax(-1), cand.argmax(-1)).astype(np.int64)


def quantize_fp4_e2m1_g32(x):
    """Per group of 32: scale 2^e with e = fp4_group_exponent(amax); code = nearest
    E2M1 value of x / 2^e (exact division by a power of two), ties to the even code,
    sign bit 3 = the sign of x (a negative value that rounds to zero is -0, as in IEEE
    rounding); E8M0 byte = e + 127. Returns (codes uint8 [..., n/2], scales uint8
    [..., n/32])."""
    x = np.asarray(x, np.float32)
    *lead, n = x.shape
    g = x.reshape(*lead, n // 32, 32).astype(np.float64)
    e = fp4_group_exponent(np.abs(g).max(axis=-1))
    y = g / (2.0 ** e)[..., None]
    mag = e2m1_nearest(y)
    code = (mag | np.where(np.signbit(y), 8, 0)).reshape(*lead, n)
    nib = code.astype(np.uint8)
    return (nib[..., 0::2] | (nib[..., 1::2] << 4)), (e + 127).astype(np.uint8)


def quantize_int8(x, scale):
    """code = clamp(rne(x / scale), -127, 127) with the cache's fixed float32 scale."""
    q = np.rint(_f32_quotient(x, scale))
    return np.clip(q, -127, 127).astype(np.int8)


def quantize_fp8_e4m3(x, scale):
    """y = x / scale (float32), saturated to [-448, 448]; the magnitude goes to the
    nearest E4M3 magnitude, ties to the even code, and the sign bit is the sign of y
    (a negative value that rounds to zero is -0, as in IEEE rounding). Returns the
    code bytes (uint8)."""
    y = np.clip(_f32_quotient(x, scale).astype(np.float64), -448.0, 448.0)
    codes = np.arange(0x7F, dtype=np.uint8)               # the finite magnitudes
    vals = decode_fp8_e4m3(codes)
    d = np.abs(np.abs(y)[..., None] - vals)
    best = d.min(axis=-1, keepdims=True)
    cand = d == best
    pref = cand & ((codes & 1) == 0)
    pick = np.where(pref.any(-1), pref.argmax(-1), cand.argmax(-1))
    return (codes[pick] | np.where(np.signbit(y), 0x80, 0)).astype(np.uint8)


# ---------------------------------------------------------------------------
# Selector scoring (§2.1 score formula; §2.3 per-block maximum).
# ---------------------------------------------------------------------------
def select_score(sel_q, sel_w, sel_k):
    """Block scores s_bar[b, blk] = max over the block's selector keys j of
    sum_h w[b,h] * ReLU(q[b,h,:] . k[b,blk,j,h,:]).

    sel_q [B][H][d_idx], sel_w [B][H], sel_k [B][nb][kpb][H][d_idx] (already decoded).
    Returns float64 [B][nb].
    """
    q = np.asarray(sel_q, dtype=np.float64)
    w = np.asarray(sel_w, dtype=np.float64)
    k = np.asarray(sel_k, dtype=np.float64)
    dots = np.einsum("bhi,bnjhi->bnjh", q, k)          # q_h . k_{h,t}
    per_key = (w[:, None, None, :] * np.maximum(dots, 0.0)).sum(axis=-1)
    return per_key.max(axis=-1)                         # max over t in the block


# ---------------------------------------------------------------------------
# Dual top-p selection (§2.3, Eq. 7 and Eq. 8).
# ---------------------------------------------------------------------------
def reserved_set(nb, n_sink, n_rec):
    """S_sink (first n_sink blocks) union S_rec (last n_rec blocks), clipped to [0, nb)."""
    sink = set(range(0, min(n_sink, nb)))
    rec = set(range(max(nb - n_rec, 0), nb))
    return sorted(sink | rec)


def select_topp_row(scores, p, K_min, K_max, n_sink, n_rec):
    """Dual top-p on one query's block scores.

    1. reserve the sink prefix and the recency suffix;
    2. softmax of the scores over the residual blocks only (Eq. 7);
    3. sort the residual blocks by score descending (lower index first on ties) and
       take the smallest prefix whose cumulative mass reaches p (the nucleus);
    4. clamp the prefix length so that |S| lies in [K_min, K_max] (Eq. 8's floor, and
       the cap), extending or cutting along the same order;
    5. S = reserved union prefix, reported in ascending order.

    Returns (sel: sorted list of block indices, info: dict of diagnostics).
    """
    s = np.asarray(scores, dtype=np.float64)
    nb = s.shape[0]
    reserved = reserved_set(nb, n_sink, n_rec)
    r = len(reserved)
    if K_max < r:
        raise ValueError("K_max smaller than the reserved set")
    rset = set(reserved)
    residual = np.array([i for i in range(nb) if i not in rset], dtype=np.int64)
    info = {"r": r, "n_res": len(residual), "k_p": 0, "k": 0, "mass": 0.0}
    if len(residual) == 0:
        info["k_p"] = 0
        return list(range(nb)), info
    sr = s[residual]
    m = sr.max()
    e = np.exp(sr - m)
    Z = e.sum()
    order = np.lexsort((residual, -sr))                 # score desc, then index asc
    n_res = len(residual)
    if p >= 1.0:
        k_p = n_res
    elif p <= 0.0:
        k_p = 0
    else:
        cum = np.cumsum(e[order])
        hit = np.nonzero(cum >= p * Z)[0]
        k_p = int(hit[0]) + 1 if len(hit) else n_res
    lo = max(0, K_min - r)
    hi = K_max - r
    k = min(max(k_p, lo), hi, n_res)
    chosen = residual[order[:k]]
    sel = sorted(set(reserved) | set(int(c) for c in chosen))
    info.update(k_p=k_p, k=k, mass=float(e[order[:k]].sum() / Z),
                cum=np.cumsum(e[order]) / Z, order=residual[order], sorted_scores=sr[order])
    return sel, info


def select_topp(scores, p, K_min, K_max, n_sink, n_rec):
    """Row-wise dual top-p over scores [B][nb]; returns a list of sorted index lists
    and a list of per-row diagnostics."""
    scores = np.asarray(scores, dtype=np.float64)
    sels, infos = [], []
    for row in scores:
        sel, info = select_topp_row(row, p, K_min, K_max, n_sink, n_rec)
        sels.append(sel)
        infos.append(info)
    return sels, infos


# ---------------------------------------------------------------------------
# Attention over the selected blocks (§2.3: the layer attends only to keys in
# blocks of S_q; one set per query, shared by every head of the layer).
# Written as dense softmax attention with -inf outside the selected keys.
# ---------------------------------------------------------------------------
def token_mask(sel, L, block):
    """Boolean [L]: True for tokens whose block is in ``sel``."""
    mask = np.zeros(L, dtype=bool)
    nbl = -(-L // block)
    for blk in sel:
        blk = int(blk)
        if 0 <= blk < nbl:
            mask[blk * block: min((blk + 1) * block, L)] = True
    return mask


def sparse_attention(q, K, V, sels, block, sm_scale, heads=None):
    """Decode attention restricted to the selected blocks.

    q [B][Hq][d]; K, V [B][Hkv][L][d]; sels[b] = block indices for query b.
    Query head hq reads KV head hq // (Hq/Hkv). Returns float64 [B][Hq][d]
    (rows not in ``heads`` are left at zero when a subset of (b, hq) is given).
    """
    q = np.asarray(q)
    B, Hq, d = q.shape
    Hkv, L = K.shape[1], K.shape[2]
    G = Hq // Hkv
    out = np.zeros((B, Hq, d), dtype=np.float64)
    for b in range(B):
        mask = token_mask(sels[b], L, block)
        if not mask.any():
            continue
        for g in range(Hkv):
            hqs = [h for h in range(g * G, (g + 1) * G) if heads is None or (b, h) in heads]
            if not hqs:
                continue
            Kg = np.asarray(K[b, g], dtype=np.float64)
            Vg = np.asarray(V[b, g], dtype=np.float64)
            for hq in hqs:
                z = (Kg @ np.asarray(q[b, hq], dtype=np.float64)) * sm_scale
                z = np.where(mask, z, -np.inf)
                w = np.exp(z - z.max())
                out[b, hq] = (w @ Vg) / w.sum()
    return out


# ---------------------------------------------------------------------------
# Prefill tile variant (§2.1: one score per query-block x key-block tile;
# §2.3 selection; causal attention within the tile).
# ---------------------------------------------------------------------------
def prefill_tile_score(sel_q, sel_w, sel_k, q_pos0, block):
    """Tile block scores for a tile of Tq consecutive queries at positions
    q_pos0 .. q_pos0+Tq-1.

    sel_q [B][Tq][H][d_idx], sel_w [B][Tq][H], sel_k [B][nb][kpb][H][d_idx].
    A block is visible to a query when its first token is at or before the query's
    position. The tile score of a block is the maximum, over the tile's queries that
    see it, of that query's block score. Returns float64 [B][nb_vis] with
    nb_vis = ceil((q_pos0 + Tq) / block).
    """
    q = np.asarray(sel_q, dtype=np.float64)
    w = np.asarray(sel_w, dtype=np.float64)
    k = np.asarray(sel_k, dtype=np.float64)
    B, Tq = q.shape[0], q.shape[1]
    nb_vis = -(-(q_pos0 + Tq) // block)
    k = k[:, :nb_vis]
    dots = np.einsum("bqhi,bnjhi->bqnjh", q, k)
    per_key = (w[:, :, None, None, :] * np.maximum(dots, 0.0)).sum(axis=-1)
    per_q = per_key.max(axis=-1)                           # [B][Tq][nb_vis]
    pos = q_pos0 + np.arange(Tq)
    first_tok = np.arange(nb_vis) * block
    visible = first_tok[None, :] <= pos[:, None]           # [Tq][nb_vis]
    per_q = np.where(visible[None], per_q, -np.inf)
    return per_q.max(axis=1)


def prefill_attention(Q, K, V, sels, block, sm_scale, q_pos0, heads=None):
    """Causal attention for a prefill tile restricted to the selected blocks.

    Q [B][Hq][Tq][d]; K, V [B][Hkv][L][d]. Query i (position q_pos0 + i) reads the
    tokens t <= q_pos0 + i whose block is selected. Returns float64 [B][Hq][Tq][d].
    """
    Q = np.asarray(Q)
    B, Hq, Tq, d = Q.shape
    Hkv, L = K.shape[1], K.shape[2]
    G = Hq // Hkv
    out = np.zeros((B, Hq, Tq, d), dtype=np.float64)
    pos = q_pos0 + np.arange(Tq)
    for b in range(B):
        sel_mask = token_mask(sels[b], L, block)
        causal = np.arange(L)[None, :] <= pos[:, None]      # [Tq][L]
        mask = causal & sel_mask[None, :]
        for g in range(Hkv):
            hqs = [h for h in range(g * G, (g + 1) * G) if heads is None or (b, h) in heads]
            if not hqs:
                continue
            Kg = np.asarray(K[b, g], dtype=np.float64)
            Vg = np.asarray(V[b, g], dtype=np.float64)
            for hq in hqs:
                z = (np.asarray(Q[b, hq], dtype=np.float64) @ Kg.T) * sm_scale   # [Tq][L]
                z = np.where(mask, z, -np.inf)
                zmax = z.max(axis=1, keepdims=True)
                has = np.isfinite(zmax)
                w = np.where(mask, np.exp(z - np.where(has, zmax, 0.0)), 0.0)
                den = w.sum(axis=1, keepdims=True)
                out[b, hq] = np.where(has, (w @ Vg) / np.where(den > 0, den, 1.0), 0.0)
    return out


def prefill_sequence(sel_q, sel_w, sel_k, Q, K, V, Tq, q_pos0, block, sm_scale, p, K_min,
                     K_max, n_sink, n_rec):
    """Sparse prefill of a whole sequence of T queries (positions q_pos0 .. q_pos0+T-1)
    cut into consecutive tiles of Tq queries (the last one shorter): for each tile, the
    tile block scores over its visible blocks (§2.1), dual top-p over them with the
    recency window ending at the tile's diagonal (§2.3, Eq. 7-8), and causal attention
    over the selected blocks. The three steps are the single-tile functions above,
    applied tile after tile.

    sel_q [B][T][H][d_idx], sel_w [B][T][H], sel_k [B][nb][kpb][H][d_idx] (decoded),
    Q [B][Hq][T][d], K, V [B][Hkv][L][d]. Returns (out float64 [B][Hq][T][d], per tile:
    the scores [B][nb_vis] and the selected sets)."""
    Q = np.asarray(Q)
    B, Hq, T, d = Q.shape
    out = np.zeros((B, Hq, T, d), dtype=np.float64)
    tiles = []
    for q0 in range(0, T, Tq):
        q1 = min(q0 + Tq, T)
        sc = prefill_tile_score(np.asarray(sel_q)[:, q0:q1], np.asarray(sel_w)[:, q0:q1],
                                sel_k, q_pos0 + q0, block)
        sets = [select_topp_row(sc[b], p, K_min, K_max, n_sink, n_rec)[0] for b in range(B)]
        out[:, :, q0:q1] = prefill_attention(Q[:, :, q0:q1], K, V, sets, block, sm_scale,
                                             q_pos0 + q0)
        tiles.append((sc, sets))
    return out, tiles

