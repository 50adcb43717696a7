"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every
symbol the header declares and nothing else under the spot_ prefix, and rejects bad
arguments before anything reaches the device. Only argument sets that fail
validation are passed here, so no kernel is ever launched."""
import ctypes
import subprocess

import pytest
import torch

from block_sparse_long_spot_amd import _lib

INVALID, UNSUPPORTED = _lib.SPOT_ERR_INVALID, _lib.SPOT_ERR_UNSUPPORTED
F32, BF16, INT4 = _lib.SPOT_F32, _lib.SPOT_BF16, _lib.SPOT_INT4_G32
INT8, FP8, FP4 = _lib.SPOT_INT8, _lib.SPOT_FP8_E4M3, _lib.SPOT_FP4_E2M1_G32


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def fake(addr=0x10000):
    """A non-null, 256-byte-aligned address that is never dereferenced."""
    return ctypes.c_void_p(addr)


def test_exports_match_header(lib):
    declared = _lib.declared_symbols()
    assert len(declared) == 11
    for name in declared:
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = sorted({ln.split()[-1] for ln in out.splitlines() if " spot_" in ln})
    assert exported == declared


def test_status_strings(lib):
    assert _lib.status_string(0) == "SPOT_OK"
    for s in (INVALID, UNSUPPORTED, _lib.SPOT_ERR_DEVICE, 12345):
        assert isinstance(_lib.status_string(s), str) and _lib.status_string(s)
    assert lib.spot_abi_version() == 3


def score(lib, **kw):
    a = dict(sel_q=fake(), q_dtype=BF16, sel_q_scale=None, sel_w=fake(), sel_k=fake(),
             sel_k_scale=None, k_dtype=BF16, scores=fake(), B=1, nb=8, kpb=1, H_idx=4,
             d_idx=64, stream=None)
    a.update(kw)
    return lib.spot_select_score(*a.values())


def test_select_score_validation(lib):
    assert score(lib, sel_q=None) == INVALID
    assert score(lib, sel_k=fake(0x10008)) == INVALID              # misaligned keys
    assert score(lib, B=0) == INVALID
    assert score(lib, nb=-1) == INVALID
    assert score(lib, kpb=0) == INVALID
    assert score(lib, q_dtype=INT4) == INVALID                      # quantised q, no scale
    assert score(lib, q_dtype=6) == INVALID
    assert score(lib, sel_q_scale=fake()) == INVALID                # scale with a bf16 query
    assert score(lib, k_dtype=7) == INVALID
    assert score(lib, k_dtype=INT4) == INVALID                      # missing scales
    assert score(lib, sel_k_scale=fake()) == INVALID                # scales with bf16 keys
    assert score(lib, k_dtype=INT4, sel_k_scale=fake(), d_idx=48) == INVALID
    assert score(lib, k_dtype=FP4, sel_k_scale=fake(), d_idx=48) == INVALID
    assert score(lib, k_dtype=INT8, sel_k_scale=fake(0x10002)) == INVALID   # fp32 scale
    assert score(lib, k_dtype=INT4, sel_k_scale=fake(0x10001)) == INVALID   # fp16 scales
    assert score(lib, d_idx=96) == UNSUPPORTED
    assert score(lib, H_idx=3) == UNSUPPORTED
    assert score(lib, H_idx=16, d_idx=64) == UNSUPPORTED            # 128 lanes per key row
    # 16 (8-bit formats) or 32 (4-bit formats) elements per lane: 128 lanes again
    assert score(lib, H_idx=32, d_idx=64, k_dtype=INT8, sel_k_scale=fake()) == UNSUPPORTED
    assert score(lib, H_idx=64, d_idx=64, k_dtype=FP4, sel_k_scale=fake()) == UNSUPPORTED


def quant(lib, **kw):
    a = dict(src=fake(), src_dtype=BF16, n_rows=4, row_len=256, fmt=INT4, codes=fake(),
             scales=fake(), tensor_scale=None, stream=None)
    a.update(kw)
    return lib.spot_quantize_selector(*a.values())


def test_quantize_selector_validation(lib):
    assert quant(lib, src=None) == INVALID
    assert quant(lib, codes=None) == INVALID
    assert quant(lib, n_rows=0) == INVALID
    assert quant(lib, row_len=48) == INVALID                        # not whole groups
    assert quant(lib, src_dtype=INT8) == INVALID
    assert quant(lib, fmt=BF16) == INVALID                          # not a quantised format
    assert quant(lib, src=fake(0x10008)) == INVALID
    assert quant(lib, codes=fake(0x10004)) == INVALID
    assert quant(lib, scales=None) == INVALID                       # INT4 writes scales
    assert quant(lib, scales=fake(0x10001)) == INVALID              # fp16 scales misaligned
    assert quant(lib, tensor_scale=fake()) == INVALID               # no tensor scale for INT4
    assert quant(lib, fmt=FP4, scales=None) == INVALID
    assert quant(lib, fmt=INT8, scales=None) == INVALID             # INT8 reads the tensor scale
    assert quant(lib, fmt=FP8, scales=None, tensor_scale=fake(0x10002)) == INVALID
    assert quant(lib, fmt=FP8, tensor_scale=fake()) == INVALID      # group scales given


def topp(lib, **kw):
    a = dict(scores=fake(), sel_idx=fake(), sel_cnt=fake(), sel_mass=None, B=2, nb=64,
             p=0.9, K_min=4, K_max=16, n_sink=1, n_rec=2, stream=None)
    a.update(kw)
    return lib.spot_select_topp(*a.values())


def test_select_topp_validation(lib):
    assert topp(lib, scores=None) == INVALID
    assert topp(lib, sel_idx=fake(0x10002)) == INVALID
    assert topp(lib, p=float("nan")) == INVALID
    assert topp(lib, p=float("inf")) == INVALID
    assert topp(lib, K_max=2) == INVALID           # reserved set (3 blocks) does not fit
    assert topp(lib, K_max=0) == INVALID
    assert topp(lib, n_sink=-1) == INVALID
    assert topp(lib, K_min=-1) == INVALID
    assert topp(lib, nb=0) == INVALID
    assert topp(lib, nb=16385, K_max=20000) == UNSUPPORTED


def attn(lib, **kw):
    a = dict(q=fake(), k=fake(), v=fake(), kv_dtype=BF16, sel_idx=fake(), sel_cnt=fake(),
             K_max=16, out=fake(), ws=fake(), ws_bytes=1 << 30, B=1, Hq=8, Hkv=2, d=128,
             L=4096, block=64, sm_scale=0.125, stream=None)
    a.update(kw)
    return lib.spot_sparse_attn(*a.values())


def test_sparse_attn_validation(lib):
    assert attn(lib, q=None) == INVALID
    assert attn(lib, ws=fake(0x10080)) == INVALID          # workspace not 256-byte aligned
    assert attn(lib, ws_bytes=100) == INVALID
    assert attn(lib, Hq=6, Hkv=4) == INVALID
    assert attn(lib, kv_dtype=INT4) == INVALID
    assert attn(lib, L=0) == INVALID
    assert attn(lib, sm_scale=float("nan")) == INVALID
    assert attn(lib, d=96) == UNSUPPORTED
    assert attn(lib, block=48) == UNSUPPORTED
    assert attn(lib, block=256) == UNSUPPORTED
    assert attn(lib, Hq=48, Hkv=3) == UNSUPPORTED           # 16 heads per KV head
    assert attn(lib, ws_bytes=4259839, B=8, Hq=32, Hkv=8, K_max=256) == INVALID   # one short


def test_sparse_attn_noalloc_validation(lib):
    """The allocation-free form checks what spot_sparse_attn checks, and refuses sizes
    whose workspace would not fit its scratch array, before any HIP call."""
    def na(**kw):
        a = dict(q=fake(), k=fake(), v=fake(), kv_dtype=BF16, sel_idx=fake(), sel_cnt=fake(),
                 K_max=16, out=fake(), B=1, Hq=8, Hkv=2, d=128, L=4096, block=64,
                 sm_scale=0.125, stream=None)
        a.update(kw)
        return lib.spot_sparse_attn_noalloc(*a.values())
    assert na(q=None) == INVALID
    assert na(out=fake(0x10008)) == INVALID
    assert na(Hq=6, Hkv=4) == INVALID
    assert na(sm_scale=float("inf")) == INVALID
    assert na(d=96) == UNSUPPORTED
    assert na(block=48) == UNSUPPORTED
    # 64 x 32 heads x 32 slots x 130 floats = 34 MB > 32 MiB
    assert _lib.spot_sparse_attn_workspace_bytes(64, 32, 8, 128, 256) > _lib.NOALLOC_SCRATCH_BYTES
    assert na(B=64, Hq=32, Hkv=8, K_max=256) == UNSUPPORTED
    assert _lib.spot_sparse_attn_workspace_bytes(30, 32, 8, 128, 256) <= \
        _lib.NOALLOC_SCRATCH_BYTES


def test_sparse_attn_workspace_follows_the_split_plan(lib):
    """fp32 partial results and (m, l) per slot, nslot slots per (query, head) as the
    split plan uses them: batch 8 at 128K (256 work-groups of 64-block runs, runs cut
    for the whole batch in up to 32 slots), batch 1 (32 runs of 8 blocks), batch 64 with
    8192 selected blocks (128 runs per query, not 128 * 64)."""
    ws = _lib.spot_sparse_attn_workspace_bytes
    assert ws(8, 32, 8, 128, 256, 64) == 8 * 32 * 32 * 130 * 4
    assert ws(1, 32, 8, 128, 256, 64) == 1 * 32 * 32 * 130 * 4
    assert ws(64, 32, 8, 128, 8192, 64) == 64 * 32 * 128 * 130 * 4
    assert ws(1, 8, 2, 64, 16, 64, torch.float32) == 1 * 8 * 4 * 66 * 4      # 4-block runs
    assert ws(1, 8, 2, 64, 8192, 64, torch.float32) == 1 * 8 * 64 * 66 * 4   # <= 64 runs
    assert ws(0, 32, 8, 128, 256) == 0
    assert ws(8, 32, 8, 128, 256, 48) == 0                                  # no kernel
    assert ws(8, 32, 8, 96, 256) == 0
    assert ws(8, 30, 8, 128, 256) == 0


def test_prefill_validation(lib):
    a = dict(sel_q=fake(), q_dtype=BF16, sel_w=fake(), sel_k=fake(), sel_k_scale=None,
             k_dtype=BF16, scores=fake(), B=1, T=128, Tq=128, q_pos0=32640, nb_cache=512,
             kpb=1, H_idx=4, d_idx=64, block=64, stream=None)
    assert lib.spot_prefill_select_score(*{**a, "nb_cache": 100}.values()) == INVALID
    assert lib.spot_prefill_select_score(*{**a, "q_pos0": -1}.values()) == INVALID
    assert lib.spot_prefill_select_score(*{**a, "T": 0}.values()) == INVALID
    assert lib.spot_prefill_select_score(*{**a, "T": 256, "Tq": 256, "q_pos0": 0}.values()) \
        == UNSUPPORTED
    assert lib.spot_prefill_select_score(*{**a, "q_dtype": F32}.values()) == UNSUPPORTED
    # a whole 32K sequence needs 512 visible blocks: more than the cache holds here
    assert lib.spot_prefill_select_score(*{**a, "T": 32768, "q_pos0": 0,
                                           "nb_cache": 511}.values()) == INVALID
    # 65536 tiles of one query exceed the grid
    assert lib.spot_prefill_select_score(*{**a, "T": 65536, "Tq": 1, "q_pos0": 0,
                                           "nb_cache": 1024}.values()) == UNSUPPORTED
    t = dict(scores=fake(), sel_idx=fake(), sel_cnt=fake(), sel_mass=None, B=1, T=32768,
             Tq=128, q_pos0=0, block=64, p=0.95, K_min=0, K_max=512, n_sink=1, n_rec=4,
             stream=None)
    assert lib.spot_prefill_select_topp(*{**t, "scores": None}.values()) == INVALID
    assert lib.spot_prefill_select_topp(*{**t, "Tq": 0}.values()) == INVALID
    assert lib.spot_prefill_select_topp(*{**t, "p": float("inf")}.values()) == INVALID
    assert lib.spot_prefill_select_topp(*{**t, "K_max": 4}.values()) == INVALID  # r = 5
    assert lib.spot_prefill_select_topp(*{**t, "T": 2 ** 21}.values()) == UNSUPPORTED
    b = dict(q=fake(), k=fake(), v=fake(), kv_dtype=BF16, sel_idx=fake(), sel_cnt=fake(),
             K_max=512, out=fake(), B=1, Hq=32, Hkv=8, T=128, Tq=128, q_pos0=32640, d=128,
             L=32768, block=64, sm_scale=0.08, stream=None)
    assert lib.spot_prefill_attn(*{**b, "q_pos0": 32700}.values()) == INVALID   # past L
    assert lib.spot_prefill_attn(*{**b, "T": 32768, "q_pos0": 1}.values()) == INVALID
    assert lib.spot_prefill_attn(*{**b, "d": 64}.values()) == UNSUPPORTED
    assert lib.spot_prefill_attn(*{**b, "kv_dtype": F32}.values()) == UNSUPPORTED


def test_read_reference_probe_validation():
    """The benchmark's read-only reference kernel lives in its own library: it exports its
    one entry point and rejects bad arguments before any launch (no GPU needed)."""
    import os
    path = os.path.join(os.path.dirname(os.path.dirname(_lib.__file__)), "libspot_probe.so")
    probe = ctypes.CDLL(path)
    f = probe.spot_probe_read_blocks
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                  ctypes.c_void_p, ctypes.c_void_p]
    p = ctypes.c_void_p(0x1000)
    assert f(None, p, 512, 256, p, None) == -1           # no buffer
    assert f(p, None, 512, 256, p, None) == -1           # no list
    assert f(p, p, 512, 256, None, None) == -1           # no sink
    assert f(p, p, 500, 256, p, None) == -1              # not a multiple of 2 * wgs
    assert f(p, p, 0, 256, p, None) == -1
    assert f(p, p, 512, 0, p, None) == -1
