"""Pins for the oracle's bf16-expert-output mode: each expert's
down-projection result y_{t,k} rounded to bf16 (round to nearest, ties to
even) before its bias and routing weight, as tpu-inference fused_moe v1
kernel.py's dynamic_ffn2 brings the down projection's results to bf16 before
they are summed (one rounding per y_{t,k}, fp32 accumulation here). Checked
against a hand-worked example, fp64 brute force with its own rounding, and
the error bound the rounding implies on real inputs."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from moe_topk_ids_amd.inputs import bf16_bits, make_biases, make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bits(a):
    return bf16_bits(torch.as_tensor(np.asarray(a, np.float32)).to(torch.bfloat16))


def _f(bits):
    return torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).float().numpy()


def _bf16_rne(v: float) -> float:
    """v rounded to 8 significant bits, ties to even (Python's round() on an
    exact fp64 multiple), for normal-range values."""
    if v == 0.0 or not math.isfinite(v):
        return v
    m, e = math.frexp(v)  # v = m * 2^e, 0.5 <= |m| < 1
    return round(m * 256.0) / 256.0 * 2.0 ** e


def test_bf16_rne_helper():
    assert _bf16_rne(1.0 + 2 ** -8) == 1.0          # tie, even stays
    assert _bf16_rne(1.0 + 3 * 2 ** -8) == 1.0 + 2 ** -6  # tie, odd rounds up
    assert _bf16_rne(0.7310585786300049) == 0.73046875
    assert _bf16_rne(-1.6136485282199706) == -1.6171875


def test_handworked_example():
    """tests/golden/moe_bf16y_handworked.json, worked by hand."""
    g = json.load(open(os.path.join(GOLDEN, "moe_bf16y_handworked.json")))
    x, w1, w2 = _bits(g["x"]), _bits(g["w1"]), _bits(g["w2"])
    tw = np.array(g["topk_weights"], np.float32)
    ids = np.array(g["topk_ids"], np.int32)
    want = np.array(g["out"], np.float32)
    for inter in (False, True):
        got = oracle.moe_forward(x, w1, w2, tw, ids, bf16_inter=inter, bf16_y=True)
        np.testing.assert_array_equal(got, want)
    # without the rounding the result is the unrounded one
    plain = oracle.moe_forward(x, w1, w2, tw, ids)
    assert not np.array_equal(plain, want)


def _brute_force(x, w1, w2, tw, ids, b2=None):
    """fp64 scalar loops from the definition, y_{t,k} rounded by _bf16_rne,
    then b2 and the weight."""
    xf, w1f, w2f = _f(x).astype(float), _f(w1).astype(float), _f(w2).astype(float)
    T, H = xf.shape
    E, I2, _ = w1f.shape
    I = I2 // 2
    K = ids.shape[1]
    out = np.zeros((T, H))
    for t in range(T):
        for k in range(K):
            e = int(ids[t, k])
            act = []
            for i in range(I):
                g = sum(xf[t, h] * w1f[e, i, h] for h in range(H))
                u = sum(xf[t, h] * w1f[e, I + i, h] for h in range(H))
                act.append(g / (1.0 + math.exp(-g)) * u)
            for h in range(H):
                y = _bf16_rne(sum(act[i] * w2f[e, h, i] for i in range(I)))
                if b2 is not None:
                    y += float(b2[e, h])
                out[t, h] += float(tw[t, k]) * y
    return out


@pytest.mark.parametrize("T,H,I,E,K,bias", [(3, 16, 8, 4, 2, False), (2, 8, 24, 5, 3, True),
                                            (4, 32, 16, 3, 1, False), (5, 24, 40, 6, 2, True)])
def test_brute_force_fp64(T, H, I, E, K, bias):
    """Nearly every output equals the brute force to fp32 rounding: only a
    y_{t,k} whose fp32 and exact values straddle a bf16 rounding boundary
    (a few in ten thousand) may round apart. A dropped or misplaced rounding
    (none, after the weight, truncation) moves most outputs by up to half a
    bf16 ulp of y and fails."""
    d = make_inputs(T, H, I, E, K, seed=T * 13 + I)
    x = _bits(_f(bf16_bits(d["hidden_states"])) * 20.0)  # silu's non-linear range
    w1, w2 = bf16_bits(d["w1"]), bf16_bits(d["w2"])
    tw, ids = d["topk_weights"].numpy(), d["topk_ids"].numpy()
    b2 = make_biases(H, I, E, seed=T)["b2"].numpy() if bias else None
    want = _brute_force(x, w1, w2, tw, ids, b2)
    got = oracle.moe_forward_act(x, w1, w2, tw, ids, b2=b2, bf16_y=True)
    scale = np.max(np.abs(want))
    close = np.abs(got - want) <= 2e-6 * scale
    assert close.mean() >= 0.95, close.mean()
    # where they differ, by at most one bf16 ulp of a y term
    assert np.max(np.abs(got - want)) <= 2.0 ** -7 * scale


def test_rounding_error_bound_on_tiny_config():
    """On the tiny workload the bf16-y output differs from the fp32 one by at
    most sum_k |w_k| * |y_k| * 2^-8 (bf16 keeps 8 significant bits: round to
    nearest moves a value by at most 2^-8 of itself) plus fp32 rounding, and
    the rounding does change most outputs."""
    T, H, I, E, K = 64, 512, 256, 8, 2
    d = make_inputs(T, H, I, E, K, seed=0)
    x, w1, w2 = bf16_bits(d["hidden_states"]), bf16_bits(d["w1"]), bf16_bits(d["w2"])
    tw, ids = d["topk_weights"].numpy(), d["topk_ids"].numpy()
    for inter in (False, True):
        a = oracle.moe_forward(x, w1, w2, tw, ids, bf16_inter=inter)
        b = oracle.moe_forward(x, w1, w2, tw, ids, bf16_inter=inter, bf16_y=True)
        bound = np.zeros((T, H))
        for k in range(K):  # |y_k| from the fp64 oracle, one slot at a time
            yk = oracle.moe_forward_f64(x, w1, w2, np.ones((T, 1)), ids[:, k:k + 1])
            bound += np.abs(tw[:, k:k + 1]) * np.abs(yk) * 2.0 ** -8 * (1 + 1e-3)
        slack = 4e-7 * np.max(np.abs(a))
        assert np.all(np.abs(b.astype(np.float64) - a) <= bound + slack)
        assert np.mean(a != b) >= 0.9
