"""Router kernel vs the router oracle: ids bit-exact, weights to fp32 rounding."""
import numpy as np
import pytest
import torch

import moe_topk_ids_amd as moe
import oracle
from gpu_helpers import assert_close, oracle_rows, require_gpu, say, shape_inputs, to_device
from moe_topk_ids_amd.inputs import SHAPES

pytestmark = pytest.mark.gpu

W_RTOL = 4e-6  # fp32 softmax: exp rounding and a different summation order


def _check(logits: np.ndarray, K: int, label: str):
    say(f"router {label}: T={logits.shape[0]} E={logits.shape[1]} K={K}")
    d = torch.from_numpy(np.ascontiguousarray(logits, np.float32)).cuda()
    for renorm in (True, False):
        w, ids = moe.moe_topk_softmax(d, K, renormalize=renorm)
        torch.cuda.synchronize()
        ww, wi = oracle.topk_softmax(logits, K, renormalize=renorm)
        np.testing.assert_array_equal(ids.cpu().numpy(), wi, err_msg=f"{label} ids")
        np.testing.assert_allclose(w.cpu().numpy(), ww, rtol=W_RTOL, atol=1e-12,
                                   err_msg=f"{label} weights")


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
    assert_close(out.cpu().numpy(), oracle_rows(ref, rows), oracle_rows(ref, rows, True),
                 "router+forward")
