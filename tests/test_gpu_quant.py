"""GPU parity of spot_quantize_selector (quantise-on-append of selector keys): codes
and scales bit for bit against the oracle's quantisers, and an append into a cache
followed by scoring."""
import numpy as np
import pytest
import torch

from block_sparse_long_spot_amd import _lib
from oracle import spot_oracle as O
from parity import assert_scores_close, decode_selector, np64, score_magnitude

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    _lib.load()


def _data(kind, n_rows, row_len, g):
    x = torch.randn(n_rows, row_len, generator=g)
    if kind == "wide":          # magnitudes spread over six decades, per group
        x = x * torch.pow(10.0, torch.rand(n_rows, row_len // 32, 1, generator=g) * 6 - 3
                          ).repeat_interleave(32, -1).reshape(n_rows, row_len)
    elif kind == "zeros":       # whole zero groups, signed zeros, tiny values
        x[:, :32] = 0.0
        x[:, 32:64] = -0.0
        x[:, 64:96] *= 1e-30
    return x


def _ties(fmt, n_rows, row_len, g):
    """Groups whose scaled values sit exactly on rounding midpoints of the format."""
    x = torch.zeros(n_rows, row_len)
    ng = row_len // 32
    if fmt == "fp4":
        mids = torch.tensor([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
        for r in range(n_rows):
            for gi in range(ng):
                e = int(torch.randint(-4, 5, (1,), generator=g))
                v = mids[torch.randint(0, 7, (32,), generator=g)]
                v = v * torch.where(torch.rand(32, generator=g) < 0.5, -1.0, 1.0)
                v[0] = 6.0                                   # fixes the group scale at 2^e
                x[r, 32 * gi:32 * gi + 32] = v * 2.0 ** e
    elif fmt == "int4":
        for r in range(n_rows):
            for gi in range(ng):
                s = 2.0 ** int(torch.randint(-4, 4, (1,), generator=g))
                k = torch.randint(-7, 7, (32,), generator=g).float() + 0.5   # halves
                k[0] = 7.0                                   # amax = 7 s: scale exact
                x[r, 32 * gi:32 * gi + 32] = k * s
    elif fmt == "int8":
        x = (torch.randint(-126, 126, (n_rows, row_len), generator=g).float() + 0.5) * 0.25
    else:  # fp8: midpoints between neighbouring E4M3 values
        vals = np.unique(O.decode_fp8_e4m3(np.arange(0x7F, dtype=np.uint8)))
        mids = torch.from_numpy((vals[1:] + vals[:-1]) / 2).float()
        x = mids[torch.randint(0, len(mids), (n_rows, row_len), generator=g)]
        x = x * torch.where(torch.rand(n_rows, row_len, generator=g) < 0.5, -1.0, 1.0)
    return x


def _oracle(fmt, x, s):
    xs = x.numpy().astype(np.float32)
    if fmt == "int4":
        return O.quantize_int4_g32(xs)
    if fmt == "fp4":
        return O.quantize_fp4_e2m1_g32(xs)
    if fmt == "int8":
        return O.quantize_int8(xs, s).view(np.uint8), None
    return O.quantize_fp8_e4m3(xs, s), None


def _run(fmt, x_dev, s_dev):
    n_rows, row_len = x_dev.shape
    if fmt in ("int4", "fp4"):
        codes = torch.full((n_rows, row_len // 2), 0xAA, dtype=torch.uint8, device=DEV)
        scales = torch.full((n_rows, row_len // 32), 0x55,
                            dtype=torch.float16 if fmt == "int4" else torch.uint8, device=DEV)
        if fmt == "int4":
            scales.fill_(-3.0)
        _lib.spot_quantize_selector(x_dev, fmt, codes, scales=scales)
        return codes, scales
    codes = torch.full((n_rows, row_len), 0xAA, dtype=torch.uint8, device=DEV)
    _lib.spot_quantize_selector(x_dev, fmt, codes, tensor_scale=s_dev)
    return codes, None


QUANT_CASES = [
    # format, source dtype, rows, row length, data
    ("int4", "f32", 64, 256, "normal"),
    ("int4", "bf16", 33, 512, "wide"),
    ("int4", "f32", 8, 128, "zeros"),
    ("int4", "f32", 16, 256, "ties"),
    ("fp4", "f32", 64, 256, "normal"),
    ("fp4", "bf16", 33, 512, "wide"),
    ("fp4", "f32", 8, 128, "zeros"),
    ("fp4", "f32", 16, 256, "ties"),
    ("int8", "f32", 64, 256, "normal"),
    ("int8", "bf16", 40, 64, "wide"),
    ("int8", "f32", 16, 256, "ties"),
    ("int8", "f32", 8, 128, "saturate"),
    ("fp8", "f32", 64, 256, "normal"),
    ("fp8", "bf16", 40, 64, "wide"),
    ("fp8", "f32", 16, 256, "ties"),
    ("fp8", "f32", 8, 128, "saturate"),
    ("fp8", "f32", 8, 128, "zeros"),
    ("fp4", "f32", 1000, 512, "normal"),                # 16000 groups: several work-groups
]


@pytest.mark.parametrize("case", QUANT_CASES, ids=lambda c: "-".join(map(str, c)))
def test_quantize_selector_bit_exact(case):
    fmt, sdt, n_rows, row_len, kind = case
    print(f"quantise case {case}", flush=True)
    g = torch.Generator().manual_seed(n_rows * 31 + row_len + len(kind))
    x = _ties(fmt, n_rows, row_len, g) if kind == "ties" else _data(
        "normal" if kind == "saturate" else kind, n_rows, row_len, g)
    if sdt == "bf16":
        x = x.bfloat16().float()
    amax = float(x.abs().max())
    s = np.float32(1.0)
    if fmt == "int8":
        s = np.float32(0.25 if kind == "ties" else amax / 127 * (0.6 if kind == "saturate" else 1))
    elif fmt == "fp8":
        s = np.float32(1.0 if kind == "ties" else amax / 448 * (0.6 if kind == "saturate" else 1))
    s_dev = torch.tensor([s], dtype=torch.float32, device=DEV)
    x_dev = x.to(DEV, torch.bfloat16 if sdt == "bf16" else torch.float32)
    codes, scales = _run(fmt, x_dev, s_dev)
    torch.cuda.synchronize()
    want_c, want_s = _oracle(fmt, x, s)
    got_c = codes.cpu().numpy()
    bad = np.nonzero(got_c != want_c)
    assert bad[0].size == 0, (f"{bad[0].size} code bytes differ, first at {bad[0][0]},"
                              f"{bad[1][0]}: {got_c[bad][0]:#x} vs {want_c[bad][0]:#x}")
    if want_s is not None:
        got_s = scales.cpu().numpy()
        if fmt == "int4":
            np.testing.assert_array_equal(got_s.view(np.uint16), want_s.view(np.uint16))
        else:
            np.testing.assert_array_equal(got_s, want_s)


@pytest.mark.parametrize("fmt", ["fp4", "int4", "fp8"])
def test_append_into_cache_then_score(fmt):
    """Decode-time append: a per-token selector cache (block 16, 4 x 128) holds 255
    quantised blocks; the 16 keys of the newest block are quantised straight into their
    rows of the cache, then the whole cache is scored and checked against the oracle."""
    nb, kpb, H, di = 256, 16, 4, 128
    g = torch.Generator(device=DEV)
    g.manual_seed(5)
    keys = torch.randn(1, nb, kpb, H, di, generator=g, device=DEV)
    s_dev = (keys.abs().amax() / 448).reshape(1).float()
    rows = keys.reshape(nb * kpb, H * di)
    if fmt in ("int4", "fp4"):
        codes = torch.zeros(nb * kpb, H * di // 2, dtype=torch.uint8, device=DEV)
        scales = torch.zeros(nb * kpb, H * di // 32,
                             dtype=torch.float16 if fmt == "int4" else torch.uint8, device=DEV)
        _lib.spot_quantize_selector(rows[:-kpb].contiguous(), fmt, codes[:-kpb], scales=scales[:-kpb])
        _lib.spot_quantize_selector(rows[-kpb:].contiguous(), fmt, codes[-kpb:], scales=scales[-kpb:])
        k_codes, k_scale = codes.view(1, nb, kpb, H, di // 2), scales.view(1, nb, kpb, H, di // 32)
    else:
        codes = torch.zeros(nb * kpb, H * di, dtype=torch.uint8, device=DEV)
        _lib.spot_quantize_selector(rows[:-kpb].contiguous(), fmt, codes[:-kpb], tensor_scale=s_dev)
        _lib.spot_quantize_selector(rows[-kpb:].contiguous(), fmt, codes[-kpb:], tensor_scale=s_dev)
        k_codes, k_scale = codes.view(torch.float8_e4m3fn).view(1, nb, kpb, H, di), s_dev
    sel_q = torch.randn(1, H, di, generator=g, device=DEV).bfloat16()
    sel_w = torch.rand(1, H, generator=g, device=DEV)
    scores = torch.empty(1, nb, device=DEV)
    _lib.spot_select_score(sel_q, sel_w, k_codes, k_scale, scores, kpb=kpb)
    torch.cuda.synchronize()
    # the oracle quantises the same keys itself and decodes its own codes
    xs = rows.cpu().numpy()
    if fmt == "int4":
        c, sc = O.quantize_int4_g32(xs)
        dec = O.dequant_int4_g32(c, sc)
    elif fmt == "fp4":
        c, sc = O.quantize_fp4_e2m1_g32(xs)
        dec = O.dequant_fp4_e2m1_g32(c, sc)
    else:
        s = s_dev.cpu().numpy()[0]
        dec = O.dequant_fp8_e4m3(O.quantize_fp8_e4m3(xs, s), s)
    dec = dec.reshape(1, nb, kpb, H, di)
    np.testing.assert_array_equal(decode_selector(k_codes, k_scale), dec)
    ref = O.select_score(np64(sel_q), np64(sel_w), dec)
    assert_scores_close(np64(scores), ref, score_magnitude(np64(sel_q), np64(sel_w), dec))
