"""Pins for the CPU oracle's forward: each test checks the oracle against
something other than itself (a hand-worked example, brute force in fp64,
an independent second definition, library routines on special cases, closed
forms and exact invariances)."""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from moe_topk_ids_amd.inputs import bf16_bits, make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bits(a):
    return bf16_bits(torch.as_tensor(np.asarray(a, np.float32)).to(torch.bfloat16))


def _f(bits):
    return torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).float().numpy()


def _rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def _inputs_np(T, H, I, E, K, seed=0):
    d = make_inputs(T, H, I, E, K, seed=seed)
    return (bf16_bits(d["hidden_states"]), bf16_bits(d["w1"]), bf16_bits(d["w2"]),
            d["topk_weights"].numpy(), d["topk_ids"].numpy())


def test_handworked_example():
    """Page definition worked by hand (tests/golden/moe_handworked.json)."""
    g = json.load(open(os.path.join(GOLDEN, "moe_handworked.json")))
    x, w1, w2 = _bits(g["x"]), _bits(g["w1"]), _bits(g["w2"])
    tw = np.array(g["topk_weights"], np.float32)
    ids = np.array(g["topk_ids"], np.int32)
    want = np.array(g["out"], np.float64)
    out64 = oracle.moe_forward_f64(x, w1, w2, tw, ids)
    np.testing.assert_allclose(out64, want, rtol=0, atol=1e-15)
    out32 = oracle.moe_forward(x, w1, w2, tw, ids)
    np.testing.assert_allclose(out32, want, rtol=2e-7, atol=0)


def _brute_force_python(x, w1, w2, tw, ids):
    """fp64 scalar loops written straight from the definition."""
    xf, w1f, w2f = _f(x).astype(float), _f(w1).astype(float), _f(w2).astype(float)
    T, H = xf.shape
    E, I2, _ = w1f.shape
    I = I2 // 2
    K = ids.shape[1]
    out = [[0.0] * H for _ in range(T)]
    for t in range(T):
        for k in range(K):
            e = int(ids[t, k])
            act = []
            for i in range(I):
                g = sum(xf[t, h] * w1f[e, i, h] for h in range(H))
                u = sum(xf[t, h] * w1f[e, I + i, h] for h in range(H))
                act.append(g / (1.0 + math.exp(-g)) * u)
            for h in range(H):
                y = sum(act[i] * w2f[e, h, i] for i in range(I))
                out[t][h] += float(tw[t, k]) * y
    return np.array(out)


@pytest.mark.parametrize("T,H,I,E,K", [(3, 16, 8, 4, 2), (2, 8, 24, 5, 3), (4, 32, 16, 3, 1)])
def test_brute_force_fp64(T, H, I, E, K):
    x, w1, w2, tw, ids = _inputs_np(T, H, I, E, K, seed=T * 7 + H)
    # Inflate x so the activations reach silu's non-linear range.
    x = _bits(_f(x) * 20.0)
    want = _brute_force_python(x, w1, w2, tw, ids)
    got64 = oracle.moe_forward_f64(x, w1, w2, tw, ids)
    np.testing.assert_allclose(got64, want, rtol=1e-12, atol=1e-14)
    got32 = oracle.moe_forward(x, w1, w2, tw, ids)
    assert _rel_l2(got32, want) < 2e-6


def _p1_layout_mirror(x, w1, w2, tw, ids):
    """Second definition: the per-token loop of tpu-inference kernel.py
    ref_moe, with its weight layout w1 (E, 2, H, I), w2 (E, I, H) obtained by
    transposing the [E,2I,H] / [E,H,I] tensors; numpy fp64 matmuls."""
    xf, w1f, w2f = _f(x).astype(np.float64), _f(w1).astype(np.float64), _f(w2).astype(np.float64)
    E, I2, H = w1f.shape
    I = I2 // 2
    w1_p1 = w1f.reshape(E, 2, I, H).transpose(0, 1, 3, 2)  # (E, 2, H, I)
    w2_p1 = w2f.transpose(0, 2, 1)  # (E, I, H)
    outs = []
    for t in range(xf.shape[0]):
        tok = xf[t:t + 1]
        acts = []
        for e in ids[t]:
            wcat = np.concatenate([w1_p1[e, 0], w1_p1[e, 1]], axis=-1)  # (H, 2I)
            gmm1 = tok @ wcat
            gate, up = gmm1[:, :I], gmm1[:, I:]
            act = gate / (1.0 + np.exp(-gate)) * up
            acts.append(act @ w2_p1[e])
        y = np.concatenate(acts, axis=0)
        outs.append(np.sum(y * tw[t].astype(np.float64)[:, None], axis=0, keepdims=True))
    return np.concatenate(outs, axis=0)


def test_second_definition_tiny_config():
    x, w1, w2, tw, ids = _inputs_np(64, 512, 256, 8, 2)
    want = _p1_layout_mirror(x, w1, w2, tw, ids)
    got64 = oracle.moe_forward_f64(x, w1, w2, tw, ids)
    assert _rel_l2(got64, want) < 1e-12
    got32 = oracle.moe_forward(x, w1, w2, tw, ids)
    assert _rel_l2(got32, want) < 1e-5
    assert np.max(np.abs(got32 - want)) < 1e-6


def test_dense_swiglu_special_case():
    """E = K = 1 with weight 1 is a dense SwiGLU MLP: torch CPU F.linear/F.silu."""
    x, w1, w2, _, _ = _inputs_np(17, 64, 48, 1, 1, seed=3)
    x = _bits(_f(x) * 10.0)
    tw = np.ones((17, 1), np.float32)
    ids = np.zeros((17, 1), np.int32)
    xt = torch.from_numpy(_f(x)).double()
    w1t = torch.from_numpy(_f(w1)[0]).double()
    w2t = torch.from_numpy(_f(w2)[0]).double()
    h = F.linear(xt, w1t)
    want = F.linear(F.silu(h[:, :48]) * h[:, 48:], w2t).numpy()
    got64 = oracle.moe_forward_f64(x, w1, w2, tw, ids)
    np.testing.assert_allclose(got64, want, rtol=1e-11, atol=1e-14)
    got32 = oracle.moe_forward(x, w1, w2, tw, ids)
    assert _rel_l2(got32, want) < 2e-6


def test_identity_experts_closed_form():
    """gate = up = w2 = identity (H = I): each expert maps x to silu(x)*x, so
    out = (sum_k w_k) * silu(x) * x elementwise."""
    T, H, E, K = 9, 16, 3, 2
    eye = np.eye(H, dtype=np.float32)
    w1 = _bits(np.stack([np.concatenate([eye, eye], 0)] * E))
    w2 = _bits(np.stack([eye] * E))
    rng = np.random.default_rng(5)
    x = _bits(rng.uniform(-6, 6, size=(T, H)).astype(np.float32))
    ids = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    tw = rng.uniform(0.1, 1.0, size=(T, K)).astype(np.float32)
    xf = _f(x).astype(np.float64)
    want = tw.astype(np.float64).sum(1, keepdims=True) * (xf / (1 + np.exp(-xf)) * xf)
    got64 = oracle.moe_forward_f64(x, w1, w2, tw, ids)
    np.testing.assert_allclose(got64, want, rtol=1e-13, atol=1e-14)
    got32 = oracle.moe_forward(x, w1, w2, tw, ids)
    np.testing.assert_allclose(got32, want, rtol=1e-6, atol=1e-7)


def test_zero_input_gives_zero():
    x, w1, w2, tw, ids = _inputs_np(8, 64, 32, 4, 2)
    x[:] = 0
    assert np.all(oracle.moe_forward(x, w1, w2, tw, ids) == 0.0)


def test_power_of_two_weight_scaling_is_exact():
    x, w1, w2, tw, ids = _inputs_np(16, 128, 64, 8, 2)
    base = oracle.moe_forward(x, w1, w2, tw, ids)
    for j in (-3, 1, 4):
        got = oracle.moe_forward(x, w1, w2, (tw * np.float32(2.0 ** j)).astype(np.float32), ids)
        assert np.array_equal(got, base * np.float32(2.0 ** j))


def test_token_permutation_permutes_rows_bitwise():
    x, w1, w2, tw, ids = _inputs_np(32, 128, 64, 8, 3)
    base = oracle.moe_forward(x, w1, w2, tw, ids)
    perm = np.random.default_rng(1).permutation(32)
    got = oracle.moe_forward(x[perm], w1, w2, tw[perm], ids[perm])
    assert np.array_equal(got, base[perm])


def test_expert_relabel_is_bitwise_invariant():
    x, w1, w2, tw, ids = _inputs_np(32, 128, 64, 8, 2)
    base = oracle.moe_forward(x, w1, w2, tw, ids)
    perm = np.random.default_rng(2).permutation(8)  # new expert j is old expert perm[j]
    inv = np.argsort(perm)
    got = oracle.moe_forward(x, w1[perm], w2[perm], tw, inv[ids].astype(np.int32))
    assert np.array_equal(got, base)


def test_linear_in_routing_weights():
    x, w1, w2, tw, ids = _inputs_np(12, 64, 32, 4, 2)
    rng = np.random.default_rng(9)
    ta = rng.uniform(0, 1, tw.shape)
    tb = rng.uniform(0, 1, tw.shape)
    fa = oracle.moe_forward_f64(x, w1, w2, ta, ids)
    fb = oracle.moe_forward_f64(x, w1, w2, tb, ids)
    fab = oracle.moe_forward_f64(x, w1, w2, ta + tb, ids)
    np.testing.assert_allclose(fab, fa + fb, rtol=1e-12, atol=1e-15)


def test_out_of_range_ids_contribute_nothing():
    x, w1, w2, tw, ids = _inputs_np(10, 64, 32, 4, 2)
    bad = ids.copy()
    bad[3, 1] = -1
    bad[7, 0] = 4
    zeroed = tw.copy()
    zeroed[3, 1] = 0
    zeroed[7, 0] = 0
    got = oracle.moe_forward(x, w1, w2, tw, bad)
    want = oracle.moe_forward(x, w1, w2, zeroed, ids)
    np.testing.assert_array_equal(got, want)


def test_bf16_rounding_matches_torch():
    """The oracle's RNE fp32->bf16 agrees with torch's conversion (library)."""
    rng = np.random.default_rng(0)
    vals = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * np.float32(3.0),
        np.array([0.0, -0.0, 1.0, np.inf, -np.inf, 1e-40, -1e-40, 3.4e38], np.float32),
        # exact ties between two bf16 neighbours, both parities
        np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8)], np.float32),
    ])
    got = oracle.f32_to_bf16(vals)
    want = bf16_bits(torch.from_numpy(vals).to(torch.bfloat16))
    np.testing.assert_array_equal(got, want)
    nan = oracle.f32_to_bf16(np.array([np.nan], np.float32))
    assert np.isnan(_f(nan)[0])


def test_bf16_intermediate_mode():
    """Rounding the activation to bf16 moves the output by about bf16's
    relative precision (2**-9 per element, averaged down by the sums)."""
    x, w1, w2, tw, ids = _inputs_np(64, 512, 256, 8, 2)
    f32 = oracle.moe_forward(x, w1, w2, tw, ids)
    b16 = oracle.moe_forward(x, w1, w2, tw, ids, bf16_inter=True)
    r = _rel_l2(b16, f32)
    assert 1e-5 < r < 4e-3


def test_slot_activation_matches_fp64_within_one_ulp():
    x, w1, w2, tw, ids = _inputs_np(16, 256, 128, 8, 2)
    act = oracle.slot_act_bf16(x, w1, ids)
    xf, w1f = _f(x).astype(np.float64), _f(w1).astype(np.float64)
    I = 128
    for f in range(16 * 2):
        t, e = f // 2, ids[f // 2, f % 2]
        g = w1f[e, :I] @ xf[t]
        u = w1f[e, I:] @ xf[t]
        want = g / (1 + np.exp(-g)) * u
        got = _f(act[f]).astype(np.float64)
        # one bf16 ulp at the value's magnitude, plus fp32-accumulation slack
        ulp = np.maximum(np.abs(want), 1e-30) * 2.0 ** -7
        assert np.all(np.abs(got - want) <= ulp + 1e-6 * np.abs(g * u).max())
