"""One decode step of one layer: the three C calls enqueued back to back on a stream."""
from __future__ import annotations

import math

import torch

from . import _lib


class DecodeBuffers:
    """Device buffers a decode step writes: scores, the selected set, the attention
    workspace and the output. Allocated once and reused across steps."""

    def __init__(self, B, nb, Hq, Hkv, d, K_max, block, out_dtype, device="cuda"):
        self.scores = torch.empty(B, nb, dtype=torch.float32, device=device)
        self.sel_idx = torch.empty(B, K_max, dtype=torch.int32, device=device)
        self.sel_cnt = torch.empty(B, dtype=torch.int32, device=device)
        self.sel_mass = torch.empty(B, dtype=torch.float32, device=device)
        ws = _lib.spot_sparse_attn_workspace_bytes(B, Hq, Hkv, d, K_max, block, out_dtype)
        if ws <= 0:
            raise ValueError("no attention kernel for these sizes")
        self.workspace = torch.empty(ws, dtype=torch.uint8, device=device)
        self.out = torch.empty(B, Hq, d, dtype=out_dtype, device=device)

    @classmethod
    def of(cls, wl, out_dtype, B=None, device="cuda"):
        """Buffers for a decode step of workload `wl` (batch B, default wl.B)."""
        return cls(wl.B if B is None else B, wl.nb, wl.Hq, wl.Hkv, wl.d, wl.K_max, wl.block,
                   out_dtype, device=device)


class DecodeStep:
    """The three calls of a decode step on fixed inputs and buffers, marshalled once
    (each call still validates its arguments and launches its kernels every time)."""

    def __init__(self, inp: dict, wl, bufs: DecodeBuffers, stream=None):
        self.calls = (
            _lib.spot_select_score(inp["sel_q"], inp["sel_w"], inp["sel_k"],
                                   inp.get("sel_k_scale"), bufs.scores, kpb=wl.kpb,
                                   stream=stream, sel_q_scale=inp.get("sel_q_scale"),
                                   prepare=True),
            _lib.spot_select_topp(bufs.scores, bufs.sel_idx, bufs.sel_cnt, bufs.sel_mass, wl.p,
                                  wl.K_min, wl.K_max, wl.n_sink, wl.n_rec, stream=stream,
                                  prepare=True),
            _lib.spot_sparse_attn(inp["q"], inp["K"], inp["V"], bufs.sel_idx, bufs.sel_cnt,
                                  bufs.out, bufs.workspace, 1.0 / math.sqrt(wl.d),
                                  block=wl.block, stream=stream, prepare=True))

    def __call__(self):
        for c in self.calls:
            c()


def decode_step(inp: dict, wl, bufs: DecodeBuffers, stream=None):
    """Score every block, select each query's block set, attend over it."""
    _lib.spot_select_score(inp["sel_q"], inp["sel_w"], inp["sel_k"], inp.get("sel_k_scale"),
                           bufs.scores, kpb=wl.kpb, stream=stream,
                           sel_q_scale=inp.get("sel_q_scale"))
    _lib.spot_select_topp(bufs.scores, bufs.sel_idx, bufs.sel_cnt, bufs.sel_mass, wl.p,
                          wl.K_min, wl.K_max, wl.n_sink, wl.n_rec, stream=stream)
    _lib.spot_sparse_attn(inp["q"], inp["K"], inp["V"], bufs.sel_idx, bufs.sel_cnt, bufs.out,
                          bufs.workspace, 1.0 / math.sqrt(wl.d), block=wl.block, stream=stream)
    return bufs.out
