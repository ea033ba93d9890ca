"""Every row of the atrex-bench #009 shapes table at full size through the
default entry point; the oracle on min(T, 256) token rows of each (all rows
of T=135, seeded samples with the first and last row otherwise)."""
import functools

import numpy as np
import pytest
import torch

import moe_topk_ids_amd as moe
from gpu_helpers import assert_close, oracle_rows, require_gpu, sample_rows, say, tight_rows
from moe_topk_ids_amd.inputs import SHAPES_TABLE, make_inputs

pytestmark = pytest.mark.gpu


@functools.lru_cache(maxsize=1)
def _group(H, I, E, K):
    T_max = max(r[0] for r in SHAPES_TABLE if r[1:5] == (H, I, E, K))
    return make_inputs(T_max, H, I, E, K, seed=11)


@pytest.mark.parametrize("row", SHAPES_TABLE, ids=[f"T{r[0]}-H{r[1]}-I{r[2]}-E{r[3]}-K{r[4]}"
                                                   for r in SHAPES_TABLE])
def test_shapes_table_row(row):
    require_gpu()
    T, H, I, E, K = row[:5]
    full = _group(H, I, E, K)
    d = {k: (v[:T] if k in ("hidden_states", "topk_weights", "topk_ids", "router_logits") else v)
         for k, v in full.items()}
    say(f"shapes-table row T={T} H={H} I={I} E={E} K={K}")
    dd = {k: v.cuda() for k, v in d.items() if k != "router_logits"}
    out = moe.moe_forward(dd["hidden_states"].contiguous(), dd["w1"], dd["w2"],
                          dd["topk_weights"].contiguous(), dd["topk_ids"].contiguous())
    torch.cuda.synchronize()
    rows = sample_rows(T, 256, seed=T)
    got = out.cpu().numpy()[rows]
    assert_close(got, oracle_rows(d, rows), tight_rows(d, rows, None), f"T={T},H={H},I={I},E={E}")
    del dd, out
