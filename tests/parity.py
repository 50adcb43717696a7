"""Comparison rules shared by the GPU parity tests (the HIP path against the oracle).

Tolerances:
  scores   |g - r| <= 1e-5 * max(|r|, A, 1e-3 * max_row |r|), A = sum_h |w_h| sum_i |q_i k_i|
  top-p    identical fp32 scores on both sides: the sets are equal, except that the
           nucleus may differ by one block when a cumulative mass at the cut lies
           within 1e-5 of p;
  end-to-end selection (each side on its own scores): reserved blocks present; every
           residual block scoring above tau + delta chosen, none below tau' - delta,
           where tau / tau' are the oracle's last chosen / first unchosen score and
           delta = 1e-5 max(|tau|, |tau'|); sizes equal, or one apart near the cut;
  outputs  recomputed by the oracle on the GPU's own set: fp32 rows within
           1e-5 * max |row|; bf16 within 2e-2 absolute and within the elementwise
           rounding bound 7.5 u S + 2 ln2 ez A + u |r| (u = 2^-8; S, A = root-sum-square
           and sum of the softmax-weighted |V|; ez = the fp32 logit error bound): a
           probabilistic bound on the bf16 rounding of the probabilities (failure
           probability 1e-12 per element), which scales with the data.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import spot_oracle as O

MASS_TOL = 1e-5


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def decode_selector(codes, scale) -> np.ndarray:
    """A selector tensor in any of the library's formats, decoded by the oracle to
    float64 (the format follows from the dtypes, as in the binding)."""
    if codes.dtype == torch.int8:
        return O.dequant_int8(codes.cpu().numpy(), scale.cpu().numpy()[0])
    if codes.dtype == torch.float8_e4m3fn:
        return O.dequant_fp8_e4m3(codes.view(torch.uint8).cpu().numpy(),
                                  scale.cpu().numpy()[0])
    if codes.dtype == torch.uint8 and scale.dtype == torch.float16:
        return O.dequant_int4_g32(codes.cpu().numpy(), scale.cpu().numpy())
    if codes.dtype == torch.uint8 and scale.dtype == torch.uint8:
        return O.dequant_fp4_e2m1_g32(codes.cpu().numpy(), scale.cpu().numpy())
    assert scale is None
    return np64(codes)


def decoded_keys(inp) -> np.ndarray:
    return decode_selector(inp["sel_k"], inp.get("sel_k_scale"))


def decoded_query(inp) -> np.ndarray:
    return decode_selector(inp["sel_q"], inp.get("sel_q_scale"))


def score_magnitude(sel_q, sel_w, keys) -> np.ndarray:
    """max_j sum_h |w_h| sum_i |q_hi k_hi|: the size of the terms a block score adds up.
    The rounding error of an fp32 evaluation is bounded by a small multiple of
    (d_idx + H_idx) * 2^-24 times this, so it sets the scale of the score tolerance."""
    q = np.abs(np.asarray(sel_q, np.float64))
    w = np.abs(np.asarray(sel_w, np.float64))
    k = np.abs(np.asarray(keys, np.float64))
    return (w[:, None, None, :] * np.einsum("bhi,bnjhi->bnjh", q, k)).sum(-1).max(-1)


def assert_scores_close(g: np.ndarray, r: np.ndarray, a: np.ndarray = None):
    """|g - r| <= 1e-5 * max(|r|, A, 1e-3 max_row |r|) with A = score_magnitude."""
    g = np.asarray(g, np.float64)
    scale = np.maximum(np.abs(r), 1e-3 * np.abs(r).max(axis=-1, keepdims=True))
    if a is not None:
        scale = np.maximum(scale, a)
    bad = np.abs(g - r) > 1e-5 * scale
    assert not bad.any(), (f"{bad.sum()} scores off; worst at {np.argwhere(bad)[:5].tolist()}: "
                           f"gpu {g[bad][:5]} oracle {r[bad][:5]}")


def gpu_sets(sel_idx: torch.Tensor, sel_cnt: torch.Tensor):
    idx = sel_idx.cpu().numpy()
    cnt = sel_cnt.cpu().numpy()
    out = []
    for b in range(idx.shape[0]):
        row = idx[b]
        c = int(cnt[b])
        assert 0 <= c <= row.shape[0]
        s = row[:c].tolist()
        assert s == sorted(set(s)), f"row {b}: not ascending / repeated: {s[:20]}"
        assert (row[c:] == -1).all(), f"row {b}: padding is not -1"
        out.append(s)
    return out


def _near_cut(info, p):
    """True when a cumulative residual mass next to the nucleus cut is within
    MASS_TOL of p, so that rounding may move the cut by one block."""
    if "cum" not in info or not (0.0 < p < 1.0):
        return False
    cum = info["cum"]
    kp = info["k_p"]
    near = False
    for j in (kp - 2, kp - 1, kp):
        if 0 <= j < len(cum) and abs(cum[j] - p) <= MASS_TOL:
            near = True
    return near


def assert_topp_unit(gset, scores_row, p, K_min, K_max, n_sink, n_rec, tag=""):
    """Both sides ran on identical fp32 scores."""
    sel, info = O.select_topp_row(np.asarray(scores_row, np.float64), p, K_min, K_max,
                                  n_sink, n_rec)
    if gset == sel:
        return
    reserved = set(O.reserved_set(len(scores_row), n_sink, n_rec))
    assert reserved <= set(gset), f"{tag}: reserved blocks missing"
    kg = len(set(gset) - reserved)
    assert abs(kg - info["k"]) == 1 and _near_cut(info, p), (
        f"{tag}: gpu |S|={len(gset)} oracle |S|={len(sel)} k_p={info['k_p']} "
        f"diff={sorted(set(gset) ^ set(sel))[:10]}")
    assert set(gset) - reserved == set(info["order"][:kg].tolist()), f"{tag}: wrong order"


def assert_selection_e2e(gset, s_oracle_row, p, K_min, K_max, n_sink, n_rec, tag=""):
    """Each side ran on its own scores (GPU fp32, oracle fp64)."""
    s = np.asarray(s_oracle_row, np.float64)
    sel, info = O.select_topp_row(s, p, K_min, K_max, n_sink, n_rec)
    if gset == sel:
        return
    nb = len(s)
    reserved = set(O.reserved_set(nb, n_sink, n_rec))
    G = set(gset)
    assert reserved <= G, f"{tag}: reserved blocks missing"
    k = info["k"]
    srt = info.get("sorted_scores")
    if srt is None:
        raise AssertionError(f"{tag}: sets differ with an empty residual")
    tau = srt[k - 1] if k > 0 else np.inf
    tau2 = srt[k] if k < len(srt) else -np.inf
    fin = [abs(x) for x in (tau, tau2) if np.isfinite(x)]
    delta = 1e-5 * max(fin) if fin else 0.0
    for blk in range(nb):
        if blk in reserved:
            continue
        if s[blk] > tau + delta:
            assert blk in G, f"{tag}: block {blk} (score {s[blk]}) above the cut is missing"
        if s[blk] < tau2 - delta:
            assert blk not in G, f"{tag}: block {blk} (score {s[blk]}) below the cut is chosen"
    kg = len(G - reserved)
    if kg != k:
        assert abs(kg - k) == 1 and _near_cut(info, p), (
            f"{tag}: gpu k={kg} oracle k={k} k_p={info['k_p']}, not near the cut")


BF16_U = 2.0 ** -8   # unit roundoff of bfloat16 (8 significant bits, round to nearest)


def _rows_np(t, b, g, tok):
    """Rows `tok` of K or V [B][Hkv][L][d] (torch tensor on any device, or numpy) for
    batch b and KV head g, as float64."""
    if isinstance(t, torch.Tensor):
        idx = torch.as_tensor(tok, dtype=torch.long, device=t.device)
        return t[b, g].index_select(0, idx).to("cpu", torch.float64).numpy()
    return np.asarray(t[b, g], np.float64)[tok]


def attention_magnitude(q, K, V, sets, block, sm_scale, rows):
    """Sizes that bound the rounding of a bf16 attention output, per (b, hq) in `rows`:
      A[j]  = sum_t w_t |V[t][j]|, w the softmax weights of the query over its selected
              tokens (the worst-case scale of a perturbation of the weights);
      S[j]  = sqrt(sum_t (w_t V[t][j])^2) (the scale of a sum of independent ones);
      ez    = bound on the fp32 error of the log2-domain logits: d * 2^-23 * sm_scale *
              log2(e) * max_t sum_i |q_i K_ti| (the fp32 accumulation of d exact bf16
              products, then the scaling) + 2^-22 max |z| log2(e).
    Only the selected tokens are gathered. Returns {(b, hq): (A [d], S [d], ez)}."""
    q = np.asarray(q, np.float64) if not isinstance(q, torch.Tensor) else np64(q)
    B, Hq, d = q.shape
    Hkv, L = K.shape[1], K.shape[2]
    G = Hq // Hkv
    nbl = -(-L // block)
    out = {}
    for (b, hq) in rows:
        tok = [t for blk in sets[b] if 0 <= blk < nbl
               for t in range(blk * block, min((blk + 1) * block, L))]
        if not tok:
            out[(b, hq)] = (np.zeros(d), np.zeros(d), 0.0)
            continue
        g = hq // G
        Kt = _rows_np(K, b, g, tok)
        Vt = _rows_np(V, b, g, tok)
        z = (Kt @ q[b, hq]) * sm_scale
        w = np.exp(z - z.max())
        w /= w.sum()
        A = w @ np.abs(Vt)
        S = np.sqrt((w * w) @ (Vt * Vt))
        l2e = 1.4426950408889634
        ez = (d * 2.0 ** -23 * sm_scale * l2e * (np.abs(Kt) @ np.abs(q[b, hq])).max()
              + 2.0 ** -22 * np.abs(z).max() * l2e)
        out[(b, hq)] = (A, S, ez)
    return out


# Probabilistic rounding-error factor (Hoeffding's inequality for a sum of independent
# zero-mean terms X_t in [-u |a_t|, u |a_t|]: P(|sum X_t| >= x) <= 2 exp(-x^2 / (2 u^2
# sum a_t^2)), so |sum X_t| <= u sqrt(sum a_t^2) sqrt(2 ln(2 / eta)) except with
# probability eta; eta = 1e-12 per element). The roundings of different probabilities
# to the nearest bf16 are taken as independent and unbiased, the model of probabilistic
# rounding-error analysis (Higham and Mary, SIAM J. Sci. Comput. 41(5), 2019).
HOEFFDING_1E12 = float(np.sqrt(2.0 * np.log(2.0 / 1e-12)))


def bf16_attention_bound(A, S, ez, r, p_terms=1):
    """Elementwise bound on |gpu - oracle| for a bf16 attention output row.

    The kernels round each probability to bf16 (relative error <= u = 2^-8) before the
    P.V product and keep fp32 everywhere else. With the row sum taken over the unrounded
    probabilities (decode, p_terms = 1) the output moves by sum_t w_t delta_t V_tj; with
    the row sum taken over the rounded ones as well (prefill, p_terms = 2) by at most
    twice that. In the worst case that is u * A; for independent unbiased roundings it
    is below u * S * sqrt(2 ln(2 / 1e-12)) except with probability 1e-12, which is the
    bound used. Errors ez in the logits change every weight by a factor within
    2^(+-ez), i.e. the normalised weights by at most 2 ln2 ez relative: 2 ln2 ez * A
    (worst case, kept as is). The final rounding to bf16 adds u |r|."""
    return (p_terms * BF16_U * HOEFFDING_1E12 * S + 2 * 0.6931471805599453 * ez * A) \
        * (1 + 1e-3) + BF16_U * np.abs(r) * (1 + BF16_U) + 1e-7


def assert_out_close(g: np.ndarray, r: np.ndarray, dtype: torch.dtype, tag="", mag=None,
                     p_terms=1):
    """fp32: max |g - r| <= 1e-5 max |row| per row. bf16: |g - r| <= 2e-2 everywhere (the
    stated tolerance) and, when `mag` (one (A, S, ez) per row, from attention_magnitude) is
    given, the elementwise rounding bound of bf16_attention_bound, which scales with the
    data: at long contexts an output element is a weighted mean of thousands of values
    and far smaller than 2e-2, so only this bound can see a lost part of the sum."""
    g = np.asarray(g, np.float64)
    if dtype == torch.float32:
        rowmax = np.abs(r).max(axis=-1, keepdims=True)
        err = np.abs(g - r)
        bad = err > 1e-5 * np.maximum(rowmax, 1e-30)
        assert not bad.any(), f"{tag}: worst rel err {(err / np.maximum(rowmax, 1e-30)).max()}"
    else:
        err = np.abs(g - r).max()
        assert err <= 2e-2, f"{tag}: max abs err {err}"
        if mag is not None:
            assert_bf16_rounding_bound(g, r, mag, p_terms, tag)


def assert_bf16_rounding_bound(g, r, mag, p_terms=1, tag=""):
    """Every element of the bf16 rows g within bf16_attention_bound of the oracle's r;
    `mag` holds one (A, S, ez) per row (attention_magnitude)."""
    g2 = np.asarray(g, np.float64).reshape(-1, np.shape(g)[-1])
    r2 = np.asarray(r, np.float64).reshape(-1, np.shape(g)[-1])
    assert len(mag) == g2.shape[0]
    for i, (A, S, ez) in enumerate(mag):
        bound = bf16_attention_bound(A, S, ez, r2[i], p_terms)
        e = np.abs(g2[i] - r2[i])
        j = int(np.argmax(e - bound))
        assert (e <= bound).all(), (
            f"{tag} row {i}: error {e[j]:.3e} above the bf16 rounding bound {bound[j]:.3e} "
            f"at element {j}")


def tile_score_magnitude(sel_q, sel_w, keys, q_pos0, block) -> np.ndarray:
    """Prefill analogue of score_magnitude: the largest term size over the tile's queries
    that see each block, [B][nb_vis]."""
    q = np.abs(np.asarray(sel_q, np.float64))
    w = np.abs(np.asarray(sel_w, np.float64))
    k = np.abs(np.asarray(keys, np.float64))
    B, Tq = q.shape[0], q.shape[1]
    nb_vis = -(-(q_pos0 + Tq) // block)
    per_key = (w[:, :, None, None, :] * np.einsum("bqhi,bnjhi->bqnjh", q, k[:, :nb_vis])).sum(-1)
    per_q = per_key.max(-1)
    return per_q.max(axis=1)
