"""The allocation-free attention entry point (spot_sparse_attn_noalloc) against the
entry point that takes a workspace (spot_sparse_attn), through the C ABI on the GPU:
identical outputs on two calls in a row, the second with a smaller input (so the scratch
array holds the first call's partial results when the second one starts), then a size
beyond the scratch array, refused before anything is launched."""
import math

import pytest
import torch

from block_sparse_long_spot_amd import _lib

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    _lib.load()


def _case(seed, B, Hq, Hkv, d, L, block, K_max, dtype):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, Hq, d, generator=g).to(dtype).to(DEV)
    K = torch.randn(B, Hkv, L, d, generator=g).to(dtype).to(DEV)
    V = torch.randn(B, Hkv, L, d, generator=g).to(dtype).to(DEV)
    nb = -(-L // block)
    idx = torch.full((B, K_max), -1, dtype=torch.int32)
    cnt = torch.zeros(B, dtype=torch.int32)
    for b in range(B):
        c = int(torch.randint(1, K_max + 1, (1,), generator=g))
        idx[b, :c] = torch.randperm(nb, generator=g)[:c].sort().values.int()
        cnt[b] = c
    return q, K, V, idx.to(DEV), cnt.to(DEV)


def _both(case, block):
    q, K, V, idx, cnt = case
    B, Hq, d = q.shape
    Hkv = K.shape[1]
    scale = 1.0 / math.sqrt(d)
    ws = torch.full((_lib.spot_sparse_attn_workspace_bytes(B, Hq, Hkv, d, idx.shape[1], block,
                                                           q.dtype),), 255, dtype=torch.uint8,
                    device=DEV)
    ref = torch.full_like(q, float("nan"))
    _lib.spot_sparse_attn(q, K, V, idx, cnt, ref, ws, scale, block=block)
    got = torch.full_like(q, float("nan"))
    _lib.spot_sparse_attn_noalloc(q, K, V, idx, cnt, got, scale, block=block)
    torch.cuda.synchronize()
    return got, ref


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_noalloc_matches_workspace_entry_point(dtype):
    big = (8, 32, 8, 128, 16384, 64, 256) if dtype == torch.bfloat16 else \
        (4, 16, 4, 128, 8192, 64, 128)
    small = (2, 8, 2, 64, 3000, 32, 40)
    for i, shape in enumerate([big, small]):
        B, Hq, Hkv, d, L, block, K_max = shape
        print(f"noalloc call {i}: {shape} {dtype}", flush=True)
        got, ref = _both(_case(100 + i, *shape, dtype), block)
        assert not torch.isnan(ref).any()
        assert torch.equal(got, ref), f"call {i}: outputs differ"


def test_noalloc_refuses_sizes_beyond_the_scratch_array():
    # 64 queries x 32 heads x 32 slots x 130 floats = 34 MB > 32 MiB: refused on the host
    B, Hq, Hkv, d, L, K_max = 64, 32, 8, 128, 64, 256
    need = _lib.spot_sparse_attn_workspace_bytes(B, Hq, Hkv, d, K_max)
    assert need > _lib.NOALLOC_SCRATCH_BYTES
    q = torch.zeros(B, Hq, d, dtype=torch.bfloat16, device=DEV)
    K = torch.zeros(B, Hkv, L, d, dtype=torch.bfloat16, device=DEV)
    idx = torch.zeros(B, K_max, dtype=torch.int32, device=DEV)
    cnt = torch.zeros(B, dtype=torch.int32, device=DEV)
    out = torch.zeros_like(q)
    with pytest.raises(_lib.SpotError) as e:
        _lib.spot_sparse_attn_noalloc(q, K, K, idx, cnt, out, 0.1)
    assert e.value.status == _lib.SPOT_ERR_UNSUPPORTED
