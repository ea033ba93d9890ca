"""Routing kernel vs the routing oracle: bit-exact on every array."""
import numpy as np
import pytest
import torch

import moe_topk_ids_amd as moe
import oracle
from gpu_helpers import require_gpu, say, shape_inputs
from moe_topk_ids_amd.inputs import SHAPES

pytestmark = pytest.mark.gpu


def _check_route(ids_np: np.ndarray, E: int, M: int, label: str):
    ids = torch.from_numpy(np.ascontiguousarray(ids_np, np.int32)).cuda()
    say(f"route {label}: T={ids_np.shape[0]} K={ids_np.shape[1]} E={E} M={M}")
    r = moe.moe_route(ids, E, M)
    torch.cuda.synchronize()
    want = oracle.route(ids_np, E, M)
    P = int(want["offsets"][-1])
    n = ids_np.size
    np.testing.assert_array_equal(r["counts"].cpu().numpy(), want["counts"], err_msg="counts")
    np.testing.assert_array_equal(r["offsets"].cpu().numpy(), want["offsets"], err_msg="offsets")
    assert int(r["num_tiles"].item()) == want["num_tiles"]
    np.testing.assert_array_equal(r["sorted"].cpu().numpy()[:P], want["sorted"], err_msg="sorted")
    np.testing.assert_array_equal(r["slot_of"].cpu().numpy()[:n], want["slot_of"], err_msg="slot_of")
    np.testing.assert_array_equal(r["tile_expert"].cpu().numpy()[:P // M], want["tile_expert"],
                                  err_msg="tile_expert")


@pytest.mark.parametrize("name", list(SHAPES))
def test_route_bitexact_on_workloads(name):
    require_gpu()
    s = SHAPES[name]
    ids = shape_inputs(name)["topk_ids"].numpy()
    M = moe.moe_m_tile(s.T, s.H, s.I, s.E, s.K)
    _check_route(ids, s.E, M, name)
    for other in (64, 128, 192):
        if other != M:
            _check_route(ids, s.E, other, f"{name} M={other}")


def _rand_ids(T, K, E, seed):
    rng = np.random.default_rng(seed)
    return np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)


@pytest.mark.parametrize("case", ["one_expert", "empty_experts", "single_token_e128",
                                  "ragged_multiblock", "k_equals_e", "out_of_range",
                                  "many_blocks", "m16", "m256", "single_wg_limit",
                                  "multi_wg_just_past", "multi_wg_out_of_range",
                                  "multi_wg_e1024"])
def test_route_edge_cases(case):
    require_gpu()
    rng = np.random.default_rng(7)
    if case == "one_expert":  # every token's first choice is expert 5
        ids = _rand_ids(3000, 2, 8, 1)
        ids[:, 0] = 5
        ids[:, 1] = np.where(ids[:, 1] == 5, 6, ids[:, 1])
        _check_route(ids, 8, 128, case)
    elif case == "empty_experts":
        ids = (_rand_ids(777, 3, 4, 2) * 5).astype(np.int32)  # only experts 0,5,10,15 of 32
        _check_route(ids, 32, 64, case)
    elif case == "single_token_e128":
        _check_route(_rand_ids(1, 8, 128, 3), 128, 128, case)
    elif case == "ragged_multiblock":
        _check_route(_rand_ids(1237, 7, 40, 4), 40, 64, case)
    elif case == "k_equals_e":
        _check_route(_rand_ids(501, 8, 8, 5), 8, 128, case)
    elif case == "out_of_range":
        ids = _rand_ids(300, 4, 16, 6)
        ids[rng.integers(0, 300, 20), rng.integers(0, 4, 20)] = -3
        ids[rng.integers(0, 300, 20), rng.integers(0, 4, 20)] = 16
        _check_route(ids, 16, 64, case)
    elif case == "single_wg_limit":  # 16384 slots, 512 experts: the one-workgroup form's limit
        _check_route(_rand_ids(2048, 8, 512, 12), 512, 64, case)
    elif case == "multi_wg_just_past":  # 16392 slots: the two-launch form
        _check_route(_rand_ids(2049, 8, 64, 13), 64, 128, case)
    elif case == "multi_wg_out_of_range":
        ids = _rand_ids(5000, 8, 64, 14)
        ids[rng.integers(0, 5000, 200), rng.integers(0, 8, 200)] = -1
        ids[rng.integers(0, 5000, 200), rng.integers(0, 8, 200)] = 64
        _check_route(ids, 64, 64, case)
    elif case == "multi_wg_e1024":  # few slots, more experts than the one-workgroup form takes
        _check_route(_rand_ids(100, 8, 1024, 15), 1024, 128, case)
    elif case == "many_blocks":  # the largest workload row on the shapes table
        _check_route(_rand_ids(45936, 8, 128, 8), 128, 128, case)
    elif case == "m16":
        _check_route(_rand_ids(333, 2, 8, 9), 8, 16, case)
    elif case == "m256":
        _check_route(_rand_ids(4000, 2, 8, 10), 8, 256, case)


def test_route_is_deterministic():
    require_gpu()
    ids = torch.from_numpy(_rand_ids(20000, 8, 128, 11)).cuda()
    a = moe.moe_route(ids, 128, 128)
    b = moe.moe_route(ids, 128, 128)
    torch.cuda.synchronize()
    for k in ("counts", "offsets", "slot_of", "num_tiles"):
        assert torch.equal(a[k], b[k]), k
    # only the rows below offsets[E] (and the tiles below num_tiles) are defined
    rows = int(a["offsets"][-1].item())
    tiles = int(a["num_tiles"].item())
    assert torch.equal(a["sorted"][:rows], b["sorted"][:rows])
    assert torch.equal(a["tile_expert"][:tiles], b["tile_expert"][:tiles])


def _random_route_cases(n: int, seed: int):
    """Seeded (T, K, E, M, kind): slot counts on both sides of the
    single-workgroup limit (16384 slots) and up to 120,000 slots, 1 to 1024
    experts, top-1 to top-8, every multiple of 16 for the row tile, and id
    distributions uniform, skewed (Zipf-like expert popularity), or
    concentrated on two experts."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        E = int(rng.choice([1, 2, 3, 8, 16, 60, 128, 256, 513, 1024]))
        K = int(rng.integers(1, min(E, 8) + 1))
        slots = int(rng.choice([rng.integers(1, 300), rng.integers(300, 16385),
                                rng.integers(16385, 120000)]))
        T = max(1, slots // K)
        M = 16 * int(rng.integers(1, 17))
        cases.append((T, K, E, M, ["uniform", "skewed", "two_experts"][i % 3]))
    return cases


@pytest.mark.parametrize("T,K,E,M,kind", _random_route_cases(24, seed=20261206))
def test_route_random_cases(T, K, E, M, kind):
    require_gpu()
    rng = np.random.default_rng(T + 13 * E + 7 * M)
    if kind == "uniform" or E <= K:
        ids = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    else:
        # distinct experts per token, drawn without replacement from a skewed
        # popularity (kind "skewed": weight 1/(rank+1); "two_experts": nearly
        # everything on experts 0 and 1)
        if kind == "skewed":
            p = 1.0 / (np.arange(E) + 1.0)
        else:
            p = np.full(E, 1e-3)
            p[:2] = 1.0
        p = p / p.sum()
        ids = np.stack([rng.choice(E, size=K, replace=False, p=p) for _ in range(T)]).astype(
            np.int32)
    _check_route(ids, E, M, f"random {kind}")
