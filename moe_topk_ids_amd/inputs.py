"""Seeded synthetic inputs for the fused MoE forward.

The recipe is the one the atrex-bench operator #009 "fused_moe" page gives
in its "Input Generation" section, drawn in the same order:

* hidden states: bf16 N(0,1) scaled by 0.1, [T, H];
* w1: bf16 N(0,1) scaled by H**-0.5, [E, 2I, H] (rows 0..I-1 gate, I..2I-1 up);
* w2: bf16 N(0,1) scaled by I**-0.5, [E, H, I];
* router logits: fp32 N(0,1) [T, E]; softmax over experts, the K largest
  probabilities (distinct experts), renormalised to sum to one; fp32 weights
  and int32 ids.

Everything is drawn on the CPU from a seeded ``torch.Generator`` so that the
same seed gives the same bits on every machine (GPU random streams differ
between devices). Normal draws are made in fp32 and rounded to bf16 before
the bf16 scaling, which is the same distribution as drawing bf16 directly. The top-K selection uses a stable descending sort, so equal
probabilities go to the lower expert id. This module is shared by the tests
and the benchmark; it holds the page's input recipe and nothing of the
forward computation itself.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Shape:
    name: str
    T: int
    H: int
    I: int
    E: int
    K: int

    @property
    def flop(self) -> int:
        """Algorithmic FLOP of one forward: 2*T*K*H*(2I) + 2*T*K*I*H."""
        return 6 * self.T * self.K * self.H * self.I


# The five workloads: a tiny case, and four rows of the atrex-bench #009
# "Shapes" table (T=4195/H=2048/I=2048/E=8/top-2; T=1/H=2048/I=768/E=128/top-8;
# T=8192/H=4096/I=384/E=128/top-8; T=15381/H=4096/I=4096/E=8/top-2).
SHAPES = {
    "tiny": Shape("tiny", 64, 512, 256, 8, 2),
    "prefill": Shape("prefill", 4195, 2048, 2048, 8, 2),
    "decode": Shape("decode", 1, 2048, 768, 128, 8),
    "wide": Shape("wide", 8192, 4096, 384, 128, 8),
    "large": Shape("large", 15381, 4096, 4096, 8, 2),
}


# Every row of the atrex-bench #009 "Shapes" table: (T, H, I, E, top_k,
# T_SOL us, T_Prod us), the two times as the page prints them for its
# "XPU-A" hardware.
SHAPES_TABLE = [
    (135, 2048, 2048, 8, 2, 38.30, 232.70),
    (277, 2048, 2048, 8, 2, 56.71, 249.80),
    (668, 2048, 2048, 8, 2, 136.79, 477.10),
    (1023, 2048, 2048, 8, 2, 208.22, 539.00),
    (1979, 2048, 2048, 8, 2, 403.02, 772.50),
    (4195, 2048, 2048, 8, 2, 851.82, 1600.0),
    (7689, 2048, 2048, 8, 2, 1560.0, 2680.0),
    (15809, 2048, 2048, 8, 2, 3200.0, 5370.0),
    (1, 2048, 768, 128, 8, 14.25, 116.90),
    (2400, 2048, 768, 128, 8, 757.05, 2160.0),
    (4195, 2048, 768, 128, 8, 1320.0, 2980.0),
    (8192, 2048, 768, 128, 8, 2590.0, 4990.0),
    (15809, 2048, 768, 128, 8, 4990.0, 9090.0),
    (25632, 2048, 768, 128, 8, 8100.0, 14480.0),
    (45936, 2048, 768, 128, 8, 14520.0, 25710.0),
    (520, 4096, 384, 128, 8, 230.33, 595.80),
    (1019, 4096, 384, 128, 8, 322.57, 882.90),
    (2044, 4096, 384, 128, 8, 646.04, 1610.0),
    (3936, 4096, 384, 128, 8, 1240.0, 2800.0),
    (8192, 4096, 384, 128, 8, 2590.0, 5690.0),
    (4098, 4096, 4096, 8, 2, 3330.0, 5330.0),
    (8179, 4096, 4096, 8, 2, 6630.0, 10100.0),
    (15381, 4096, 4096, 8, 2, 12480.0, 18640.0),
]


def topk_routing(logits: torch.Tensor, K: int):
    """Softmax over experts, K largest (ties to the lower id), renormalised."""
    probs = logits.float().softmax(dim=-1)
    vals, idx = torch.sort(probs, dim=-1, descending=True, stable=True)
    w = vals[:, :K]
    w = (w / w.sum(dim=-1, keepdim=True)).to(torch.float32)
    return w.contiguous(), idx[:, :K].to(torch.int32).contiguous()


def _randn_bf16(shape, g: torch.Generator) -> torch.Tensor:
    """N(0,1) rounded to bf16 (drawn in fp32: several times faster on the CPU
    than drawing bf16 directly, same distribution)."""
    return torch.randn(shape, dtype=torch.float32, generator=g).to(torch.bfloat16)


def make_inputs(T: int, H: int, I: int, E: int, K: int, seed: int = 0) -> dict:
    """CPU tensors: hidden bf16 [T,H], w1 bf16 [E,2I,H], w2 bf16 [E,H,I],
    topk_weights fp32 [T,K], topk_ids int32 [T,K], router_logits fp32 [T,E]."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    hidden = _randn_bf16((T, H), g) * 0.1
    w1 = _randn_bf16((E, 2 * I, H), g) * H ** (-0.5)
    w2 = _randn_bf16((E, H, I), g) * I ** (-0.5)
    logits = torch.randn(T, E, dtype=torch.float32, generator=g)
    tw, ids = topk_routing(logits, K)
    return {"hidden_states": hidden, "w1": w1, "w2": w2, "topk_weights": tw,
            "topk_ids": ids, "router_logits": logits}


def make_biases(H: int, I: int, E: int, seed: int = 0) -> dict:
    """Seeded fp32 expert biases (CPU): b1 [E, 2I] (gate biases, then up
    biases) N(0,1)*0.1, the spread of the gate/up projections under the
    input recipe above; b2 [E, H] N(0,1)*0.01, about that of one expert's
    down projection. The pages give no generator for biases."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed + 1000003)
    b1 = torch.randn(E, 2 * I, dtype=torch.float32, generator=g) * 0.1
    b2 = torch.randn(E, H, dtype=torch.float32, generator=g) * 0.01
    return {"b1": b1.contiguous(), "b2": b2.contiguous()}


def quantize_fp8_blocks(w: torch.Tensor, block: int):
    """Synthetic sub-channel-quantised weights from bf16 weights [..., N, C]
    (C the contraction axis): each run of `block` consecutive elements along
    C gets the fp32 scale max|w| / 448, and the values w / scale are rounded
    to OCP FP8 E4M3 (largest finite value 448). Returns (codes uint8
    [..., N, C], scales fp32 [..., N, C/block])."""
    *lead, n, c = w.shape
    wb = w.float().reshape(*lead, n, c // block, block)
    amax = wb.abs().amax(dim=-1, keepdim=True)
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    q = (wb / scale).to(torch.float8_e4m3fn).reshape(*lead, n, c)
    return q.view(torch.uint8).contiguous(), scale.squeeze(-1).contiguous()


def make_fp8_weights(d: dict, block: int = 256) -> dict:
    """FP8 E4M3 versions of an input set's w1 and w2 with per-block scales
    along the contraction axis (H for w1, I for w2)."""
    w1q, w1s = quantize_fp8_blocks(d["w1"], block)
    w2q, w2s = quantize_fp8_blocks(d["w2"], block)
    return {"w1q": w1q, "w1s": w1s, "w2q": w2q, "w2s": w2s, "block": block}


def make_shape_inputs(name: str, seed: int = 0) -> dict:
    s = SHAPES[name]
    return make_inputs(s.T, s.H, s.I, s.E, s.K, seed=seed)


def bf16_bits(t: torch.Tensor):
    """Raw bf16 bits of a CPU bf16 tensor as a numpy uint16 array."""
    import numpy as np

    assert t.dtype == torch.bfloat16
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)
