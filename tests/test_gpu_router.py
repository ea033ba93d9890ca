"""Router kernel vs the router oracle: ids bit-exact, weights to fp32 rounding."""
import numpy as np
import pytest
import torch

import moe_topk_ids_amd as moe
import oracle
from gpu_helpers import (assert_close, oracle_rows, require_gpu, say, shape_inputs, tight_rows,
                         to_device)
from moe_topk_ids_amd.inputs import SHAPES

pytestmark = pytest.mark.gpu


def _gpu_sum_depth(E: int) -> int:
    """Roundings on the longest path of the router kernel's exp sum: each
    token's group of G lanes holds EPL logits per lane (4 up to 64 experts,
    8 up to 128, else 16; G the smallest power of two with EPL*G >= E); a
    lane adds its terms in order, then log2(G) levels of a tree over the
    group."""
    epl = 4 if E <= 64 else 8 if E <= 128 else 16
    G = 1
    while epl * G < E:
        G *= 2
    return min(epl, E) - 1 + G.bit_length() - 1


def ulp_bound(E: int, K: int, renormalize: bool) -> int:
    """Largest ulp distance the two fp32 routers can show on one weight.

    With u = 2^-24, exp taken as within 2 ulp (4u) on the GPU and 1 ulp (2u)
    in the oracle (same argument l - max on both sides), and a relative
    difference r being under r/u ulps:
    - unnormalised p = exp / denominator: the denominator sums E terms, in
      order in the oracle ((E-1)u) and along the GPU kernel's tree
      (_gpu_sum_depth(E) u); one division each. Bound:
      (4 + 4 + depth + 1)u + (2 + 2 + E - 1 + 1)u.
    - renormalised w = p_k / sum_j p_j: the denominator is a common factor
      and cancels; left are the exps, two divisions and a K-term sum (any
      order: at most K-1 roundings), (2 eps + (K+2)u) per side: (2K+16)u.
    Two more ulps cover the second-order terms.
    """
    if renormalize:
        return 2 * K + 16 + 2
    return E + _gpu_sum_depth(E) + 13 + 2


def _ulp_distance(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """ulps between non-negative finite fp32 values (their bit patterns are
    ordered like the values)."""
    ia = np.ascontiguousarray(a, np.float32).view(np.int32).astype(np.int64)
    ib = np.ascontiguousarray(b, np.float32).view(np.int32).astype(np.int64)
    return np.abs(ia - ib)


def _check(logits: np.ndarray, K: int, label: str):
    T, E = logits.shape
    d = torch.from_numpy(np.ascontiguousarray(logits, np.float32)).cuda()
    for renorm in (True, False):
        w, ids = moe.moe_topk_softmax(d, K, renormalize=renorm)
        torch.cuda.synchronize()
        ww, wi = oracle.topk_softmax(logits, K, renormalize=renorm)
        np.testing.assert_array_equal(ids.cpu().numpy(), wi, err_msg=f"{label} ids")
        got = w.cpu().numpy()
        assert np.all(got >= 0) and np.all(np.isfinite(got)), label
        dist = int(_ulp_distance(got, ww).max()) if got.size else 0
        bound = ulp_bound(E, K, renorm)
        say(f"router {label}: T={T} E={E} K={K} renormalize={renorm}: max ulp distance "
            f"{dist} (bound {bound})")
        assert dist <= bound, f"{label}: {dist} ulps > {bound}"


@pytest.mark.parametrize("name", list(SHAPES))
def test_router_on_workload_logits(name):
    require_gpu()
    s = SHAPES[name]
    _check(shape_inputs(name)["router_logits"].numpy(), s.K, name)


@pytest.mark.parametrize("T,E,K,kind", [
    (777, 40, 5, "normal"), (100, 1024, 32, "normal"), (64, 1000, 7, "normal"),
    (300, 8, 8, "normal"), (50, 1, 1, "normal"), (513, 64, 3, "ties"), (200, 130, 4, "ties"),
    (128, 16, 4, "neg_inf"), (45936, 128, 8, "normal"),
])
def test_router_edge_cases(T, E, K, kind):
    require_gpu()
    rng = np.random.default_rng(T * 7 + E)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    if kind == "ties":  # few distinct values: many exact ties
        logits = np.round(logits * 2) / 2
    elif kind == "neg_inf":  # some experts impossible, still enough finite ones
        logits[:, ::4] = -np.inf
    _check(logits, K, f"{kind}")


def _random_router_cases(n: int, seed: int):
    """Seeded (T, E, K, kind): expert counts on both sides of every layout
    boundary of the kernel (4, 8 or 16 logits per lane; 1 to 64 lanes per
    token; E a multiple of the lanes' vector width or not), top-1 to top-32,
    1 to 5000 tokens, half of them with many exact ties."""
    rng = np.random.default_rng(seed)
    es = [2, 3, 4, 5, 7, 8, 9, 15, 16, 17, 31, 33, 63, 64, 65, 96, 127, 128, 129, 200, 255, 256,
          257, 384, 511, 512, 513, 700, 1023, 1024]
    cases = []
    for i in range(n):
        E = int(es[i % len(es)])
        K = int(rng.integers(1, min(E, 32) + 1))
        T = int(rng.integers(1, 5000))
        cases.append((T, E, K, "ties" if i % 2 else "normal"))
    return cases


@pytest.mark.parametrize("T,E,K,kind", _random_router_cases(30, seed=20261205))
def test_router_random_cases(T, E, K, kind):
    require_gpu()
    rng = np.random.default_rng(T * 31 + E * 7 + K)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    if kind == "ties":
        logits = np.round(logits * 2) / 2
    _check(logits, K, f"random {kind}")


def test_router_then_forward():
    """Logits -> GPU router -> GPU forward equals logits -> oracle router ->
    oracle forward, on the tiny workload."""
    require_gpu()
    d = dict(shape_inputs("tiny"))
    dd = to_device(d)
    w, ids = moe.moe_topk_softmax(dd["router_logits"], SHAPES["tiny"].K)
    out = moe.moe_forward(dd["hidden_states"], dd["w1"], dd["w2"], w, ids)
    torch.cuda.synchronize()
    ow, oi = oracle.topk_softmax(d["router_logits"].numpy(), SHAPES["tiny"].K)
    ref = dict(d, topk_weights=torch.from_numpy(ow), topk_ids=torch.from_numpy(oi))
    rows = np.arange(SHAPES["tiny"].T)
    assert_close(out.cpu().numpy(), oracle_rows(ref, rows), tight_rows(ref, rows, None),
                 "router+forward")
