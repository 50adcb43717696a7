"""ctypes binding to libspot.so: one Python function per C entry point, same names.

Argument marshalling only: every function takes torch tensors that already live on
the GPU, checks their dtype/shape/contiguity against the C ABI's layout, and passes
raw pointers and the current torch stream to the library. No computation happens
here and there is no fallback: if the library or a GPU is missing, calls raise.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libspot.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "spot.h")

SPOT_OK, SPOT_ERR_INVALID, SPOT_ERR_UNSUPPORTED, SPOT_ERR_DEVICE = 0, -1, -2, -3
SPOT_F32, SPOT_BF16, SPOT_INT4_G32, SPOT_INT8, SPOT_FP8_E4M3, SPOT_FP4_E2M1_G32 = range(6)
ABI_VERSION = 3

_lib = None


class SpotError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status_string(status)} ({status})")


def load() -> ctypes.CDLL:
    """Load libspot.so (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m block_sparse_long_spot_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.spot_select_score.argtypes = [vp, i, vp, vp, vp, vp, i, vp, i, i, i, i, i, vp]
    lib.spot_select_score.restype = i
    lib.spot_quantize_selector.argtypes = [vp, i, i, i, i, vp, vp, vp, vp]
    lib.spot_quantize_selector.restype = i
    lib.spot_select_topp.argtypes = [vp, vp, vp, vp, i, i, f, i, i, i, i, vp]
    lib.spot_select_topp.restype = i
    lib.spot_sparse_attn_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
    lib.spot_sparse_attn_workspace_bytes.restype = sz
    lib.spot_sparse_attn.argtypes = [vp, vp, vp, i, vp, vp, i, vp, vp, sz, i, i, i, i, i, i, f,
                                     vp]
    lib.spot_sparse_attn.restype = i
    lib.spot_sparse_attn_noalloc.argtypes = [vp, vp, vp, i, vp, vp, i, vp, i, i, i, i, i, i, f,
                                             vp]
    lib.spot_sparse_attn_noalloc.restype = i
    lib.spot_prefill_select_score.argtypes = [vp, i, vp, vp, vp, i, vp, i, i, i, i, i, i, i, i,
                                              i, vp]
    lib.spot_prefill_select_score.restype = i
    lib.spot_prefill_select_topp.argtypes = [vp, vp, vp, vp, i, i, i, i, i, f, i, i, i, i, vp]
    lib.spot_prefill_select_topp.restype = i
    lib.spot_prefill_attn.argtypes = [vp, vp, vp, i, vp, vp, i, vp, i, i, i, i, i, i, i, i, i,
                                      f, vp]
    lib.spot_prefill_attn.restype = i
    lib.spot_status_string.argtypes = [i]
    lib.spot_status_string.restype = ctypes.c_char_p
    lib.spot_abi_version.argtypes = []
    lib.spot_abi_version.restype = i
    if lib.spot_abi_version() != ABI_VERSION:
        raise RuntimeError(f"{LIB_PATH} has ABI {lib.spot_abi_version()}, this binding "
                           f"expects {ABI_VERSION}: rebuild it")
    _lib = lib
    return lib


def declared_symbols() -> list:
    """Names of every function the C header declares."""
    text = open(HEADER_PATH).read()
    return sorted(set(re.findall(r"SPOT_API\s+[\w\s\*]+?\b(spot_\w+)\s*\(", text)))


def status_string(status: int) -> str:
    return load().spot_status_string(int(status)).decode()


def _check(fn: str, status: int):
    if status != SPOT_OK:
        raise SpotError(fn, status)


class Prepared:
    """One library call with its arguments marshalled once (pointers, sizes, stream).
    Calling it issues the same C call again, argument checks and launches included,
    without re-reading the tensors: for a caller that repeats a call on the same
    buffers, as a decode loop does. The tensors must stay alive and in place."""

    __slots__ = ("name", "fn", "args", "keep")

    def __init__(self, name: str, args: tuple, keep: tuple = ()):
        self.name, self.fn, self.args, self.keep = name, getattr(load(), name), args, keep

    def __call__(self):
        st = self.fn(*self.args)
        if st != SPOT_OK:
            raise SpotError(self.name, st)


def _issue(name: str, args: tuple, prepare: bool, keep: tuple = ()):
    """Call entry point `name` with `args`, or return it as a Prepared call."""
    if prepare:
        return Prepared(name, args, keep)
    _check(name, getattr(load(), name)(*args))


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors passed to libspot must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors passed to libspot must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SPOT_F32
    if t.dtype == torch.bfloat16:
        return SPOT_BF16
    raise ValueError(f"unsupported dtype {t.dtype}")


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def selector_format(codes: torch.Tensor, scale: Optional[torch.Tensor]):
    """The C ABI format code of a selector tensor and how many elements one stored
    element of its last axis holds, from the torch dtypes:
      float32 / bfloat16, no scale               -> SPOT_F32 / SPOT_BF16
      int8 codes, float32 scale [1]              -> SPOT_INT8
      float8_e4m3fn codes, float32 scale [1]     -> SPOT_FP8_E4M3
      uint8 (two 4-bit codes), float16 scales    -> SPOT_INT4_G32
      uint8 (two 4-bit codes), uint8 E8M0 scales -> SPOT_FP4_E2M1_G32"""
    dt = codes.dtype
    if dt in (torch.float32, torch.bfloat16):
        if scale is not None:
            raise ValueError("fp32/bf16 selector tensors take no scale")
        return _dtype_code(codes), 1
    if scale is None:
        raise ValueError(f"a {dt} selector tensor needs its scale tensor")
    if dt in (torch.int8, torch.float8_e4m3fn):
        if scale.dtype != torch.float32 or scale.numel() != 1:
            raise ValueError("INT8 / FP8 selector tensors take one float32 scale")
        return (SPOT_INT8 if dt == torch.int8 else SPOT_FP8_E4M3), 1
    if dt == torch.uint8 and scale.dtype == torch.float16:
        return SPOT_INT4_G32, 2
    if dt == torch.uint8 and scale.dtype == torch.uint8:
        return SPOT_FP4_E2M1_G32, 2
    raise ValueError(f"unsupported selector format {dt} with scale {scale.dtype}")


def spot_select_score(sel_q, sel_w, sel_k, sel_k_scale, scores, kpb: int = 1, stream=None,
                      sel_q_scale=None, prepare: bool = False):
    """scores[B][nb] <- selector block scores. sel_q [B][H][d_idx] and sel_k
    [B][nb][kpb][H][d_idx] in any selector format (see selector_format; 4-bit formats
    store d_idx/2 bytes per row), each with its scale tensor or None. prepare=True
    returns the call as a Prepared object instead of issuing it."""
    B, H = sel_w.shape
    q_fmt, q_per = selector_format(sel_q, sel_q_scale)
    k_fmt, k_per = selector_format(sel_k, sel_k_scale)
    d_idx = sel_q.shape[-1] * q_per
    assert sel_q.shape == (B, H, d_idx // q_per) and sel_k.shape[-1] * k_per == d_idx
    nb = scores.shape[1]
    assert scores.dtype == torch.float32 and sel_w.dtype == torch.float32
    return _issue("spot_select_score",
                  (_ptr(sel_q), q_fmt, _ptr(sel_q_scale), _ptr(sel_w), _ptr(sel_k),
                   _ptr(sel_k_scale), k_fmt, _ptr(scores), B, nb, kpb, H, d_idx,
                   _stream(stream)), prepare, (sel_q, sel_q_scale, sel_w, sel_k, sel_k_scale,
                                               scores))


_FORMATS = {"int4": SPOT_INT4_G32, "fp4": SPOT_FP4_E2M1_G32, "int8": SPOT_INT8,
            "fp8": SPOT_FP8_E4M3}


def spot_quantize_selector(src, fmt: str, codes, scales=None, tensor_scale=None,
                           stream=None):
    """Encode src [n_rows][row_len] (fp32/bf16, row_len % 32 == 0) into codes (uint8
    [n_rows][row_len/2] for "int4"/"fp4", [n_rows][row_len] int8 / float8_e4m3fn for
    "int8"/"fp8") and, for the group formats, scales [n_rows][row_len/32] (fp16 for
    "int4", uint8 E8M0 for "fp4"); the 8-bit formats read the cache's fp32 scale [1]."""
    n_rows, row_len = src.shape
    st = load().spot_quantize_selector(_ptr(src), _dtype_code(src), n_rows, row_len,
                                       _FORMATS[fmt], _ptr(codes), _ptr(scales),
                                       _ptr(tensor_scale), _stream(stream))
    _check("spot_quantize_selector", st)


def spot_select_topp(scores, sel_idx, sel_cnt, sel_mass, p: float, K_min: int, K_max: int,
                     n_sink: int, n_rec: int, stream=None, prepare: bool = False):
    """sel_idx[B][K_max] (ascending, -1 padded), sel_cnt[B], optional sel_mass[B]."""
    B, nb = scores.shape
    assert sel_idx.dtype == torch.int32 and sel_idx.shape == (B, K_max)
    assert sel_cnt.dtype == torch.int32
    return _issue("spot_select_topp",
                  (_ptr(scores), _ptr(sel_idx), _ptr(sel_cnt), _ptr(sel_mass), B, nb, float(p),
                   K_min, K_max, n_sink, n_rec, _stream(stream)), prepare,
                  (scores, sel_idx, sel_cnt, sel_mass))


def spot_sparse_attn_workspace_bytes(B: int, Hq: int, Hkv: int, d: int, K_max: int,
                                     block: int = 64, dtype=torch.bfloat16) -> int:
    """Bytes of workspace spot_sparse_attn needs for these arguments (0 when they are
    invalid or unsupported); dtype is that of q, K and V."""
    code = SPOT_BF16 if dtype == torch.bfloat16 else SPOT_F32
    return int(load().spot_sparse_attn_workspace_bytes(B, Hq, Hkv, d, K_max, block, code))


def spot_sparse_attn(q, k_cache, v_cache, sel_idx, sel_cnt, out, workspace, sm_scale: float,
                     block: int = 64, stream=None, prepare: bool = False):
    """out[B][Hq][d] <- attention of q over the selected blocks of K/V [B][Hkv][L][d]."""
    B, Hq, d = q.shape
    Hkv, L = k_cache.shape[1], k_cache.shape[2]
    K_max = sel_idx.shape[1]
    return _issue("spot_sparse_attn",
                  (_ptr(q), _ptr(k_cache), _ptr(v_cache), _dtype_code(q), _ptr(sel_idx),
                   _ptr(sel_cnt), K_max, _ptr(out), _ptr(workspace),
                   workspace.numel() * workspace.element_size(), B, Hq, Hkv, d, L, block,
                   float(sm_scale), _stream(stream)), prepare,
                  (q, k_cache, v_cache, sel_idx, sel_cnt, out, workspace))


NOALLOC_SCRATCH_BYTES = 32 << 20   # SPOT_NOALLOC_SCRATCH_BYTES


def spot_sparse_attn_noalloc(q, k_cache, v_cache, sel_idx, sel_cnt, out, sm_scale: float,
                             block: int = 64, stream=None):
    """spot_sparse_attn without a workspace argument: the library's per-GPU scratch array
    holds the partial results, and nothing is allocated. Calls that may overlap on one
    GPU must be ordered by the caller."""
    B, Hq, d = q.shape
    Hkv, L = k_cache.shape[1], k_cache.shape[2]
    K_max = sel_idx.shape[1]
    st = load().spot_sparse_attn_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _dtype_code(q),
                                         _ptr(sel_idx), _ptr(sel_cnt), K_max, _ptr(out), B, Hq,
                                         Hkv, d, L, block, float(sm_scale), _stream(stream))
    _check("spot_sparse_attn_noalloc", st)


def _tiles(T: int, Tq) -> tuple:
    Tq = T if Tq is None else int(Tq)
    return Tq, -(-T // Tq)


def spot_prefill_select_score(sel_q, sel_w, sel_k, scores, q_pos0: int, block: int = 64,
                              kpb: int = 1, Tq: Optional[int] = None, stream=None,
                              sel_k_scale=None):
    """scores[B][n_tiles][nb_seq] (or [B][nb_seq] for one tile) <- tile block scores of
    the T queries of sel_q [B][T][H][d_idx] (bf16) at positions q_pos0.., in tiles of Tq
    (default: one tile of T). sel_k [B][nb_cache][kpb][H][..] in bf16 or a quantised
    selector format with its scale tensor (see selector_format)."""
    B, T, H, d_idx = sel_q.shape
    Tq, n_tiles = _tiles(T, Tq)
    nb_cache = sel_k.shape[1]
    nb_seq = -(-(q_pos0 + T) // block)
    assert scores.numel() == B * n_tiles * nb_seq and scores.dtype == torch.float32
    k_fmt, k_per = selector_format(sel_k, sel_k_scale)
    assert sel_k.shape[-1] * k_per == d_idx
    st = load().spot_prefill_select_score(_ptr(sel_q), _dtype_code(sel_q), _ptr(sel_w),
                                          _ptr(sel_k), _ptr(sel_k_scale), k_fmt, _ptr(scores),
                                          B, T, Tq, q_pos0, nb_cache, kpb, H, d_idx, block,
                                          _stream(stream))
    _check("spot_prefill_select_score", st)


def spot_prefill_select_topp(scores, sel_idx, sel_cnt, sel_mass, p: float, K_min: int,
                             K_max: int, n_sink: int, n_rec: int, q_pos0: int, T: int,
                             Tq: Optional[int] = None, block: int = 64, stream=None):
    """Per-tile dual top-p: sel_idx [B][n_tiles][K_max], sel_cnt [B][n_tiles]; each tile
    sees its own visible blocks, recency ending at its diagonal."""
    B = scores.shape[0]
    Tq, n_tiles = _tiles(T, Tq)
    nb_seq = -(-(q_pos0 + T) // block)
    assert scores.numel() == B * n_tiles * nb_seq
    assert sel_idx.dtype == torch.int32 and sel_idx.numel() == B * n_tiles * K_max
    assert sel_cnt.dtype == torch.int32 and sel_cnt.numel() == B * n_tiles
    st = load().spot_prefill_select_topp(_ptr(scores), _ptr(sel_idx), _ptr(sel_cnt),
                                         _ptr(sel_mass), B, T, Tq, q_pos0, block, float(p),
                                         K_min, K_max, n_sink, n_rec, _stream(stream))
    _check("spot_prefill_select_topp", st)


def spot_prefill_attn(q, k_cache, v_cache, sel_idx, sel_cnt, out, q_pos0: int,
                      sm_scale: float, block: int = 64, Tq: Optional[int] = None, stream=None):
    """out[B][Hq][T][d] <- causal attention of every tile over its selected blocks
    (sel_idx [B][n_tiles][K_max] or [B][K_max] for one tile)."""
    B, Hq, T, d = q.shape
    Tq, n_tiles = _tiles(T, Tq)
    Hkv, L = k_cache.shape[1], k_cache.shape[2]
    K_max = sel_idx.shape[-1]
    assert sel_idx.numel() == B * n_tiles * K_max and sel_cnt.numel() == B * n_tiles
    st = load().spot_prefill_attn(_ptr(q), _ptr(k_cache), _ptr(v_cache), _dtype_code(q),
                                  _ptr(sel_idx), _ptr(sel_cnt), K_max, _ptr(out), B, Hq, Hkv,
                                  T, Tq, q_pos0, d, L, block, float(sm_scale), _stream(stream))
    _check("spot_prefill_attn", st)


def spot_abi_version() -> int:
    return int(load().spot_abi_version())
