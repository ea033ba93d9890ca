"""Pins for the oracle's forward with sub-channel-quantised weights (the later
tpu-inference fused_moe kernel.py's ref_moe with w1_scale / w2_scale): the
FP8 E4M3 decode against torch's float8_e4m3fn, and reductions to the
unquantised forward where the dequantised weights are exact."""
import numpy as np
import pytest
import torch

import oracle
from moe_topk_ids_amd.inputs import bf16_bits, make_biases, make_fp8_weights, make_inputs


def test_fp8_decode_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.fp8_e4m3_to_f32(codes)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF]) and got[0x7E] == 448.0


def _codes(rng, shape):
    c = rng.integers(0, 256, size=shape, dtype=np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x38  # no NaN codes (0x38 is 1.0)
    # keep magnitudes moderate: exponent field at most 9 (|v| < 8)
    e = (c >> 3) & 15
    c = np.where(e > 9, (c & 0x87) | (9 << 3), c).astype(np.uint8)
    return c


def _dequant_bf16(codes, scales, block):
    v = torch.from_numpy(codes).view(torch.float8_e4m3fn).float()
    s = torch.from_numpy(scales).repeat_interleave(block, dim=-1)
    w = (v * s).to(torch.bfloat16)
    assert torch.equal(w.float(), v * s), "dequantised weights must be bf16-exact here"
    return bf16_bits(w)


@pytest.mark.parametrize("block", [128, 256])
@pytest.mark.parametrize("act", ["silu", "swigluoai"])
def test_power_of_two_scales_equal_unquantised_forward(block, act):
    """With per-block scales 2^k every dequantised weight is exact in fp32
    and in bf16, so the quantised forward must give the unquantised
    forward's bits on those weights; a scale applied to the wrong block or
    column changes the result."""
    T, H, I, E, K = 9, 512, 256, 4, 2
    rng = np.random.default_rng(block)
    d = make_inputs(T, H, I, E, K, seed=13)
    w1q, w2q = _codes(rng, (E, 2 * I, H)), _codes(rng, (E, H, I))
    w1s = (2.0 ** rng.integers(-8, -3, size=(E, 2 * I, H // block))).astype(np.float32)
    w2s = (2.0 ** rng.integers(-8, -3, size=(E, H, I // block))).astype(np.float32)
    b = make_biases(H, I, E, seed=13)
    kw = dict(act=act, b1=b["b1"].numpy(), b2=b["b2"].numpy())
    if act == "swigluoai":
        kw.update(alpha=1.702, limit=0.5)
    x, tw, ids = bf16_bits(d["hidden_states"]), d["topk_weights"].numpy(), d["topk_ids"].numpy()
    got = oracle.moe_forward_q(x, w1q, w1s, w2q, w2s, block, tw, ids, **kw)
    want = oracle.moe_forward_act(x, _dequant_bf16(w1q, w1s, block), _dequant_bf16(w2q, w2s, block),
                                  tw, ids, **kw)
    assert np.array_equal(got, want)
    # the same holds in bf16-intermediate mode
    got16 = oracle.moe_forward_q(x, w1q, w1s, w2q, w2s, block, tw, ids, bf16_inter=True, **kw)
    want16 = oracle.moe_forward_act(x, _dequant_bf16(w1q, w1s, block),
                                    _dequant_bf16(w2q, w2s, block), tw, ids, bf16_inter=True, **kw)
    assert np.array_equal(got16, want16)


def test_generator_quantisation_is_close_to_the_bf16_weights():
    """The synthetic FP8 weights (max-abs scaling per block of 256) stay
    within E4M3's relative precision of the bf16 weights they come from, and
    the quantised forward within a few percent of the bf16 forward."""
    T, H, I, E, K = 16, 512, 256, 4, 2
    d = make_inputs(T, H, I, E, K, seed=14)
    q = make_fp8_weights(d, 256)
    deq = (q["w1q"].view(torch.float8_e4m3fn).float()
           * q["w1s"].repeat_interleave(256, dim=-1))
    err = (deq - d["w1"].float()).abs() / d["w1"].float().abs().clamp_min(1e-30)
    big = d["w1"].float().abs() > q["w1s"].repeat_interleave(256, dim=-1) * 2 ** -6
    assert float(err[big].max()) <= 2 ** -4 + 1e-6  # half an ulp of a 3-bit mantissa
    x, tw, ids = bf16_bits(d["hidden_states"]), d["topk_weights"].numpy(), d["topk_ids"].numpy()
    got = oracle.moe_forward_q(x, q["w1q"].numpy(), q["w1s"].numpy(), q["w2q"].numpy(),
                               q["w2s"].numpy(), 256, tw, ids)
    want = oracle.moe_forward(x, bf16_bits(d["w1"]), bf16_bits(d["w2"]), tw, ids)
    assert np.linalg.norm(got - want) / np.linalg.norm(want) < 0.06
