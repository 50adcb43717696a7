"""Seeded synthetic inputs for the SpotAttention decode and prefill paths.

This module builds inputs only. It holds none of the method's arithmetic: it
computes no selector score, no selection and no attention. The oracle tests, the
GPU parity tests and the benchmark all draw their inputs from here, so the oracle
and the HIP path always read the same arrays.

Workloads stand in for the paper's Qwen3-8B decode measurements (SpotAttention:
Plug-In Block-Sparse Routing for Pretrained Long-Context Transformers, Table 1),
whose activations, KV caches and trained selectors are not available. Every tensor
is drawn from a torch generator seeded with ``seed``, in a fixed order:
selector query, selector weights, selector keys, q, K, V, then the planted /
Zipf structure.

Layouts (row-major, innermost last):
  sel_q  [B][H_idx][d_idx]           (decode)   or [B][Tq][H_idx][d_idx] (prefill)
  sel_w  [B][H_idx] fp32             (decode)   or [B][Tq][H_idx]        (prefill)
  sel_k  [B][nb][kpb][H_idx][d_idx]  fp32/bf16, int8 or float8_e4m3fn codes (with one
         fp32 scale [1]), or 4-bit codes [B][nb][kpb][H_idx][d_idx/2] uint8 with
         scales [B][nb][kpb][H_idx][d_idx/32]: fp16 for INT4, E8M0 bytes for FP4
  sel_q  may be quantised the same ways (Workload.sel_q_dtype)
  q      [B][Hq][d]                  (decode)   or [B][Hq][Tq][d]        (prefill)
  K, V   [B][Hkv][L][d]
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    L: int
    block: int
    H_idx: int
    d_idx: int
    kpb: int
    dtype: str            # "f32" or "bf16": q, K, V, selector query and selector keys
    sel_k_dtype: str      # "f32", "bf16", "int8", "fp8", "int4" or "fp4"
    p: float
    K_min: int
    K_max: int
    n_sink: int
    n_rec: int
    structure: str        # "planted", "zipf", "none"
    n_plant: int = 0
    zipf_s: float = 1.1
    zipf_spread: Optional[tuple] = None   # (s_lo, s_hi) across the batch
    prefill_Tq: int = 0   # > 0: a prefill tile of Tq queries ending at position L-1
    seed: int = 42
    sel_q_dtype: Optional[str] = None     # quantised selector query (None: dtype)

    @property
    def nb(self) -> int:
        return -(-self.L // self.block)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def q_pos0(self) -> int:
        return self.L - self.prefill_Tq

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads: a small fp32 case, the Qwen3-8B-shaped layer at 32K, the
# same layer at 128K (batch 1 and 8), the 128K batch-8 case with an INT4 selector
# cache, and a 128-query prefill tile at 32K. A sixth uses the paper's own selector
# geometry and inference settings (Appendix A, Table 3): 16-token blocks, one selector
# key per token (4 heads x 128), sink 128 tokens, recency 256 tokens, a K_min floor of
# 512 tokens, dual top-p at p = 0.9 and no cap on |S|.
WORKLOADS = {
    "c1_small_f32": Workload(
        "c1_small_f32", B=1, Hq=8, Hkv=2, d=64, L=4096, block=64, H_idx=4, d_idx=32, kpb=1,
        dtype="f32", sel_k_dtype="f32", p=0.9, K_min=4, K_max=16, n_sink=1, n_rec=2,
        structure="planted", n_plant=4, seed=42),
    "c2_32k_b4": Workload(
        "c2_32k_b4", B=4, Hq=32, Hkv=8, d=128, L=32768, block=64, H_idx=4, d_idx=64, kpb=1,
        dtype="bf16", sel_k_dtype="bf16", p=0.95, K_min=16, K_max=128, n_sink=1, n_rec=4,
        structure="planted", n_plant=5, seed=43),
    "c3_128k_b1": Workload(
        "c3_128k_b1", B=1, Hq=32, Hkv=8, d=128, L=131072, block=64, H_idx=4, d_idx=64, kpb=1,
        dtype="bf16", sel_k_dtype="bf16", p=0.95, K_min=16, K_max=256, n_sink=1, n_rec=4,
        structure="zipf", zipf_s=1.1, seed=44),
    "c3_128k_b8": Workload(
        "c3_128k_b8", B=8, Hq=32, Hkv=8, d=128, L=131072, block=64, H_idx=4, d_idx=64, kpb=1,
        dtype="bf16", sel_k_dtype="bf16", p=0.95, K_min=16, K_max=256, n_sink=1, n_rec=4,
        structure="zipf", zipf_s=1.1, seed=44),
    "c4_128k_b8_int4": Workload(
        "c4_128k_b8_int4", B=8, Hq=32, Hkv=8, d=128, L=131072, block=64, H_idx=4, d_idx=64,
        kpb=1, dtype="bf16", sel_k_dtype="int4", p=0.95, K_min=16, K_max=256, n_sink=1,
        n_rec=4, structure="zipf", zipf_s=1.1, seed=45),
    "c5_prefill_32k": Workload(
        "c5_prefill_32k", B=1, Hq=32, Hkv=8, d=128, L=32768, block=64, H_idx=4, d_idx=64,
        kpb=1, dtype="bf16", sel_k_dtype="bf16", p=0.95, K_min=0, K_max=512, n_sink=1,
        n_rec=4, structure="none", prefill_Tq=128, seed=46),
    "page_128k_b1": Workload(
        "page_128k_b1", B=1, Hq=32, Hkv=8, d=128, L=131072, block=16, H_idx=4, d_idx=128,
        kpb=16, dtype="bf16", sel_k_dtype="bf16", p=0.9, K_min=32, K_max=8192, n_sink=8,
        n_rec=16, structure="zipf", zipf_s=1.1, seed=47),
}


def _tdtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def reserved_blocks(nb: int, n_sink: int, n_rec: int) -> list:
    """Block indices held back from the nucleus: the first n_sink and the last n_rec."""
    res = set(range(min(n_sink, nb))) | set(range(max(nb - n_rec, 0), nb))
    return sorted(res)


def quantize_int4_g32(x: torch.Tensor):
    """Symmetric INT4 with one fp16 scale per 32 consecutive elements of the last axis.

    scale = fp16(amax / 7); code = clamp(round_half_even(x / scale), -8, 7); codes are
    two's-complement nibbles, even element in the low nibble. Returns (codes uint8
    [..., n/2], scales fp16 [..., n/32]). Storage is 4 + 16/32 = 4.5 bits per element.
    """
    *lead, n = x.shape
    assert n % 32 == 0
    xg = x.float().reshape(*lead, n // 32, 32)
    amax = xg.abs().amax(dim=-1)
    scale16 = (amax / 7.0).to(torch.float16)
    s = scale16.float().unsqueeze(-1)
    q = torch.where(s > 0, torch.round(xg / torch.where(s > 0, s, torch.ones_like(s))),
                    torch.zeros_like(xg))
    q = q.clamp(-8, 7).to(torch.int32).reshape(*lead, n)
    nib = (q & 0xF).to(torch.uint8)
    codes = nib[..., 0::2] | (nib[..., 1::2] << 4)
    return codes.contiguous(), scale16.contiguous()


def quantize_int8_tensor(x: torch.Tensor):
    """Symmetric INT8 with one fp32 scale for the whole tensor: scale = amax / 127,
    code = clamp(round_half_even(x / scale), -127, 127). 8 bits per element. Returns
    (codes int8, scale float32 [1])."""
    amax = x.float().abs().amax()
    scale = (amax / 127.0).clamp_min(torch.finfo(torch.float32).tiny).reshape(1)
    codes = torch.round(x.float() / scale).clamp(-127, 127).to(torch.int8)
    return codes.contiguous(), scale.float().contiguous()


def quantize_fp8_e4m3_tensor(x: torch.Tensor):
    """FP8 E4M3 with one fp32 scale for the whole tensor: scale = amax / 448 (the
    largest finite E4M3 value), codes = x / scale rounded by torch's float8_e4m3fn
    cast (done on the CPU). 8 bits per element. Returns (codes float8_e4m3fn,
    scale float32 [1])."""
    amax = x.float().abs().amax()
    scale = (amax / 448.0).clamp_min(torch.finfo(torch.float32).tiny).reshape(1)
    codes = (x.float() / scale).cpu().to(torch.float8_e4m3fn).to(x.device)
    return codes.contiguous(), scale.float().contiguous()


_FP4_MAGS = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def quantize_fp4_e2m1_g32(x: torch.Tensor):
    """FP4 E2M1 with one E8M0 (power-of-two) scale per 32 consecutive elements of the
    last axis: scale = 2^ceil(log2(amax / 6)) so that |x| / scale <= 6, code = the
    nearest E2M1 value of x / scale (sign in bit 3), two codes per byte with the even
    element in the low nibble. 4 + 8/32 = 4.25 bits per element. Returns (codes uint8
    [..., n/2], scales uint8 [..., n/32] holding the biased exponent)."""
    *lead, n = x.shape
    assert n % 32 == 0
    xg = x.float().reshape(*lead, n // 32, 32)
    amax = xg.abs().amax(dim=-1)
    e = torch.ceil(torch.log2(torch.where(amax > 0, amax / 6.0, torch.ones_like(amax))))
    e = e.clamp(-127, 127)
    scale = torch.pow(2.0, e).unsqueeze(-1)
    y = (xg / scale).abs()
    mags = torch.tensor(_FP4_MAGS, device=x.device)
    mids = (mags[1:] + mags[:-1]) / 2
    mag_code = torch.bucketize(y, mids)                    # index of the nearest magnitude
    sign = ((xg < 0) & (mag_code > 0)).to(torch.int64) << 3
    nib = (mag_code | sign).reshape(*lead, n).to(torch.uint8)
    codes = nib[..., 0::2] | (nib[..., 1::2] << 4)
    scales = (e + 127).to(torch.uint8)
    return codes.contiguous(), scales.contiguous()


def quantize_selector(x: torch.Tensor, fmt: str):
    """Encode x in one of the selector-cache formats; returns (codes, scale or None)."""
    if fmt in ("f32", "bf16"):
        return x.to(_tdtype(fmt)).contiguous(), None
    return {"int4": quantize_int4_g32, "int8": quantize_int8_tensor,
            "fp8": quantize_fp8_e4m3_tensor, "fp4": quantize_fp4_e2m1_g32}[fmt](x)


def make_inputs(wl: Workload, device="cpu", seed: Optional[int] = None,
                B: Optional[int] = None) -> dict:
    """Draw one batch of inputs for workload ``wl`` on ``device``.

    Planted blocks ("planted"): n_plant residual blocks per batch element get selector
    keys 3*sel_q (every selector head) and backbone keys 3*(mean of the group's q) for
    every token of the block. Zipf ("zipf"): every residual block gets a rank r from a
    random permutation and a target selector score t = s*ln(n_res/r) >= 0, realised by
    k_h = (t / sum_h w_h) * q_h / |q_h|^2 plus N(0, I) noise projected orthogonal to q_h,
    so that softmax over residual blocks of the targets is Zipf(s).
    """
    seed = wl.seed if seed is None else seed
    B = wl.B if B is None else B
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    f32 = torch.float32
    nb, kpb, H, di = wl.nb, wl.kpb, wl.H_idx, wl.d_idx
    Tq = wl.prefill_Tq

    def randn(*shape):
        return torch.randn(*shape, generator=gen, device=device, dtype=f32)

    if Tq:
        sel_q = randn(B, Tq, H, di)
        sel_w = randn(B, Tq, H).abs()
    else:
        sel_q = randn(B, H, di)
        sel_w = randn(B, H).abs()
    sel_k = randn(B, nb, kpb, H, di)
    q = randn(B, wl.Hq, Tq, wl.d) if Tq else randn(B, wl.Hq, wl.d)
    dt = _tdtype(wl.dtype)
    K = torch.empty(B, wl.Hkv, wl.L, wl.d, device=device, dtype=dt)
    V = torch.empty(B, wl.Hkv, wl.L, wl.d, device=device, dtype=dt)
    for b in range(B):      # chunked draw keeps host memory at one batch element of fp32
        K[b] = randn(wl.Hkv, wl.L, wl.d).to(dt)
    for b in range(B):
        V[b] = randn(wl.Hkv, wl.L, wl.d).to(dt)

    reserved = set(reserved_blocks(nb, wl.n_sink, wl.n_rec))
    residual = torch.tensor([i for i in range(nb) if i not in reserved], dtype=torch.long)
    planted = []
    if wl.structure == "planted" and not Tq:
        qd = q.to(dt).float()
        for b in range(B):
            perm = torch.randperm(len(residual), generator=gen, device=device).cpu()
            blks = residual[perm[: wl.n_plant]].sort().values
            planted.append(blks.tolist())
            gq = qd[b].reshape(wl.Hkv, wl.G, wl.d).mean(dim=1)          # [Hkv][d]
            for blk in blks.tolist():
                sel_k[b, blk, :, :, :] = 3.0 * sel_q[b].to(dt).float()
                t0, t1 = blk * wl.block, min((blk + 1) * wl.block, wl.L)
                K[b, :, t0:t1, :] = (3.0 * gq).to(dt).unsqueeze(1)
    elif wl.structure == "zipf" and not Tq:
        n_res = len(residual)
        qd = sel_q.to(dt).float() if wl.sel_k_dtype != "f32" else sel_q
        for b in range(B):
            if wl.zipf_spread is not None and B > 1:
                s_lo, s_hi = wl.zipf_spread
                s_b = s_lo + (s_hi - s_lo) * b / (B - 1)
            else:
                s_b = wl.zipf_s
            perm = torch.randperm(n_res, generator=gen, device=device).cpu()
            rank = torch.empty(n_res, dtype=f32)
            rank[perm] = torch.arange(1, n_res + 1, dtype=f32)
            t = (s_b * torch.log(n_res / rank)).to(device)                # [n_res]
            wsum = sel_w[b].sum()
            qh = qd[b]                                                    # [H][di]
            qn2 = (qh * qh).sum(-1, keepdim=True)                         # [H][1]
            noise = sel_k[b, residual.to(device)]                         # [n_res][kpb][H][di]
            proj = (noise * qh).sum(-1, keepdim=True) / qn2
            noise = noise - proj * qh
            keys = (t / wsum).view(n_res, 1, 1, 1) * (qh / qn2) + noise
            sel_k[b, residual.to(device)] = keys
    out = {"sel_w": sel_w, "q": q.to(dt), "K": K, "V": V, "planted": planted}
    if wl.sel_q_dtype is None:
        out["sel_q"], out["sel_q_scale"] = sel_q.to(dt), None
    else:
        out["sel_q"], out["sel_q_scale"] = quantize_selector(sel_q, wl.sel_q_dtype)
    out["sel_k"], out["sel_k_scale"] = quantize_selector(sel_k, wl.sel_k_dtype)
    return out
