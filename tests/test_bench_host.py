"""Host-side checks of bench.py: the algorithmic byte counts behind the roofline and
%-of-peak figures, and the one-GPU contract. No GPU needed."""
import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from block_sparse_long_spot_amd import workloads as W  # noqa: E402


def test_attention_and_step_bytes_128k_batch8():
    """128K context, batch 8, 256 selected 64-token blocks per query: K and V of 8 KV
    heads x 128 dims in bf16, plus q and out, plus the bf16 selector keys (4 x 64 per
    block) and the selector query and weights."""
    wl = W.WORKLOADS["c3_128k_b8"]
    tokens = 8 * 256 * 64
    b = bench.byte_budget(wl, 8, tokens)
    attn = tokens * 8 * 128 * 2 * 2 + 8 * 32 * 128 * 2 * 2
    assert b["attn"] == attn == 537_001_984
    sel_keys = 8 * 2048 * 1 * 4 * 64 * 2
    sel_query = 8 * 4 * (64 * 2 + 4)
    assert b["step"] == sel_keys + sel_query + attn == 545_394_816


def test_int4_selector_bytes():
    """INT4 codes are half a byte per element plus one fp16 scale per 32 elements."""
    wl = W.WORKLOADS["c4_128k_b8_int4"]
    b = bench.byte_budget(wl, 8, 0)
    n_el = 8 * 2048 * 4 * 64
    assert b["step"] - b["attn"] == n_el // 2 + n_el // 32 * 2 + 8 * 4 * (64 * 2 + 4)


def test_selected_tokens_counts_ragged_block_and_ignores_padding():
    """A selected last block that extends past L counts only its tokens below L;
    entries past sel_cnt and out-of-range entries are not counted."""
    L, block = 1000, 64                      # 16 blocks, the last one holds 40 tokens
    idx = torch.tensor([[0, 15, 3, -1], [15, 99, 7, 7]], dtype=torch.int32)
    cnt = torch.tensor([3, 2], dtype=torch.int32)
    assert bench.selected_tokens(idx, cnt, L, block) == (64 + 40 + 64) + (40 + 0)


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""
