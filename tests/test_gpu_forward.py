"""Fused forward on the GPU vs the CPU oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import moe_topk_ids_amd as moe
import oracle
from gpu_helpers import (REL_L2_BF16_INTER, assert_close, cpu_inputs, oracle_rows,
                         random_shapes, rel_l2, require_gpu, sample_rows, say, shape_inputs,
                         tight_rows, to_device, y_bf16_for)
from moe_topk_ids_amd.inputs import SHAPES, Shape, bf16_bits

pytestmark = pytest.mark.gpu

PATHS = {
    "slot": moe.FLAG_FORCE_GROUPED,
    "atomic": moe.FLAG_FORCE_GROUPED | moe.FLAG_ATOMIC_COMBINE,
    "decode": moe.FLAG_FORCE_DECODE,
    "small_batch": moe.FLAG_FORCE_SMALL_BATCH,
}


def _run(dd, flags):
    out = moe.moe_forward(dd["hidden_states"], dd["w1"], dd["w2"], dd["topk_weights"],
                          dd["topk_ids"], flags=flags)
    torch.cuda.synchronize()
    return out.cpu().numpy()


# Token rows per workload checked against the oracle: every row of tiny,
# prefill and decode; 1024 seeded rows (first and last included) of wide and
# large, which reach every row tile and every tile window of the persistent
# schedule (wide: ~1090 row tiles of 64 rows, each holding slots of ~64
# different tokens; large: ~124 tiles of 256 rows, 2048 slots sampled).
SAMPLES = {"tiny": 64, "prefill": 4195, "decode": 1, "wide": 1024, "large": 1024}


@pytest.mark.parametrize("name", list(SHAPES))
def test_forward_matches_oracle(name):
    """Every combine path at the workload's full size against the oracle on
    all token rows (tiny, prefill, decode) or 1024 seeded rows (wide, large)."""
    require_gpu()
    s = SHAPES[name]
    d = shape_inputs(name)
    dd = to_device(d)
    rows = sample_rows(s.T, SAMPLES[name], seed=1)
    want = oracle_rows(d, rows)
    tight = {}  # bf16 activation, expert outputs bf16 or fp32 as the path stores them
    for path in ("default", "slot", "fp32_y", "atomic"):
        fl = {"default": None, "fp32_y": PATHS["slot"] | moe.FLAG_FP32_Y}.get(path, PATHS.get(path))
        yb = y_bf16_for(d, fl)
        if yb not in tight:
            tight[yb] = oracle_rows(d, rows, bf16_inter=True, bf16_y=yb)
        say(f"forward {name} path={path} bf16_y={yb}")
        got = _run(dd, fl)
        assert_close(got[rows], want, tight[yb], f"{name}/{path}")
    del dd


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill"])
def test_decode_path_matches_oracle(name):
    """The weight-streaming path on workloads it does not take by default too."""
    require_gpu()
    s = SHAPES[name]
    d = shape_inputs(name)
    if s.T > 256:  # keep the per-slot path's work small: leading tokens only
        d = {k: (v[:256] if k in ("hidden_states", "topk_weights", "topk_ids", "router_logits")
                 else v) for k, v in d.items()}
    dd = to_device(d)
    say(f"decode path on {name}")
    got = _run(dd, moe.FLAG_FORCE_DECODE)
    rows = sample_rows(got.shape[0], 64, seed=2)
    assert_close(got[rows], oracle_rows(d, rows), tight_rows(d, rows, moe.FLAG_FORCE_DECODE),
                 f"decode-path/{name}")


# leading tokens per workload for the expert-deduplicated path (T*K <= 1024)
SB_TOKENS = {"tiny": 64, "prefill": 512, "decode": 1, "wide": 128, "large": 96}


@pytest.mark.parametrize("name", list(SHAPES))
def test_small_batch_path_matches_oracle(name):
    """Each routed expert's rows streamed once for all of its slots: every
    workload's leading tokens, every gate/up and down kernel variant."""
    require_gpu()
    s = SHAPES[name]
    n = SB_TOKENS[name]
    d = {k: (v[:n] if k in ("hidden_states", "topk_weights", "topk_ids", "router_logits")
             else v) for k, v in shape_inputs(name).items()}
    assert moe.moe_path(n, s.H, s.I, s.E, s.K, moe.FLAG_FORCE_SMALL_BATCH) == \
        moe.PATH_SMALL_BATCH
    dd = to_device(d)
    say(f"small-batch path on {name} (T={n})")
    got = _run(dd, moe.FLAG_FORCE_SMALL_BATCH)
    rows = sample_rows(n, 64, seed=3)
    assert_close(got[rows], oracle_rows(d, rows), tight_rows(d, rows, moe.FLAG_FORCE_SMALL_BATCH),
                 f"small-batch/{name}")
    # the same slots on the per-token path: equal up to the order of the
    # fp32 dot products inside each row
    other = _run(dd, moe.FLAG_FORCE_DECODE)
    r = rel_l2(got, other)
    say(f"small-batch vs per-token path: rel-L2 {r:.2e}")
    assert r <= 2e-3


def test_small_batch_repeated_and_shared_experts():
    """Every token routes to the same two experts (1024 slots on one expert
    pair), and repeated ids inside a token (a precondition violation whose
    result is still the weighted sum, linear in the weights)."""
    require_gpu()
    d = dict(cpu_inputs(512, 256, 384, 16, 2, seed=11))
    ids = d["topk_ids"].clone()
    ids[:, 0] = 5
    ids[:, 1] = 12
    ids[7, 1] = 5  # token 7 routes twice to expert 5
    d["topk_ids"] = ids.contiguous()
    rows = np.arange(512)
    got = _run(to_device(d), moe.FLAG_FORCE_SMALL_BATCH)
    assert_close(got, oracle_rows(d, rows), tight_rows(d, rows, moe.FLAG_FORCE_SMALL_BATCH),
                 "small-batch/shared")


# (workload, token rows checked): the forward's gate/up tiles 128x128
# (tiny), 192x256 (prefill), 64x256 (wide) and 64x128 (the shapes-table row
# T=135, H=I=2048, E=8, top-2)
INTER_CASES = {"tiny": 64, "prefill": 1024, "wide": 512, "t135": 135}


@pytest.mark.parametrize("name", list(INTER_CASES))
def test_intermediate_matches_oracle(name):
    """GEMM1 + SiLU intermediate (the forward's own gate/up tile) vs the
    oracle's per-slot bf16 activation: at most one bf16 ulp apart, nearly all
    identical."""
    require_gpu()
    if name == "t135":
        s = Shape("t135", 135, 2048, 2048, 8, 2)
        d = cpu_inputs(s.T, s.H, s.I, s.E, s.K, seed=135)
    else:
        s = SHAPES[name]
        d = shape_inputs(name)
    dd = to_device(d)
    M = moe.moe_m_tile(s.T, s.H, s.I, s.E, s.K)
    say(f"intermediate {name} M={M}")
    r = moe.moe_route(dd["topk_ids"], s.E, M)
    act = moe.moe_gemm1_silu(dd["hidden_states"], dd["w1"], r, s.K, M)
    torch.cuda.synchronize()
    slot_of = r["slot_of"].cpu().numpy()
    rows = sample_rows(s.T, INTER_CASES[name], seed=3)
    slots = (rows[:, None] * s.K + np.arange(s.K)[None, :]).ravel()
    got = act.cpu().view(torch.int16).numpy().view(np.uint16)[slot_of[slots]]
    sub = {k: d[k] for k in d}
    want = oracle.slot_act_bf16(bf16_bits(sub["hidden_states"])[rows], bf16_bits(sub["w1"]),
                                sub["topk_ids"].numpy()[rows])
    gf = torch.from_numpy(got.view(np.int16)).view(torch.bfloat16).float().numpy()
    wf = torch.from_numpy(want.view(np.int16)).view(torch.bfloat16).float().numpy()
    # one bf16 ulp is at most 2**-7 of the value; a little absolute slack
    # covers values that round from near zero on either side
    tol = 2.0 ** -7 * np.maximum(np.abs(gf), np.abs(wf)) + 1e-7
    exact = float(np.mean(got == want))
    say(f"  identical {exact:.4f}, max |diff| {np.max(np.abs(gf - wf)):.3e}")
    assert np.all(np.abs(gf - wf) <= tol)
    assert exact >= 0.97
    # pad rows of the intermediate are zero
    offs = r["offsets"].cpu().numpy()
    counts = r["counts"].cpu().numpy()
    a16 = act.cpu().view(torch.int16).numpy()
    for e in range(s.E):
        pad = a16[offs[e] + counts[e]:offs[e + 1]]
        assert np.all(pad == 0)


def test_slot_path_is_deterministic_and_permutation_invariant():
    require_gpu()
    d = shape_inputs("prefill")
    dd = to_device(d)
    a = _run(dd, PATHS["slot"])
    b = _run(dd, PATHS["slot"])
    assert np.array_equal(a, b)
    perm = torch.from_numpy(np.random.default_rng(4).permutation(SHAPES["prefill"].T))
    pd = dict(dd)
    for k in ("hidden_states", "topk_weights", "topk_ids"):
        pd[k] = dd[k][perm.cuda()].contiguous()
    c = _run(pd, PATHS["slot"])
    assert np.array_equal(c, a[perm.numpy()])


@pytest.mark.parametrize("T,H,I,E,K", [
    (135, 2048, 2048, 8, 2),  # the shapes-table row: 16 stages per split
    (96, 1024, 640, 8, 2),    # 5 stages per split: an odd count through the GEMM loop
])
def test_split_down_projection(T, H, I, E, K):
    """Few tokens per expert: the down projection's contraction is split and
    the combine adds the partial rows in a fixed order. Against the oracle on
    every row; bitwise run-to-run and under token permutation (the split is
    the same for every row)."""
    require_gpu()
    n = T * K
    slot_ws = moe.moe_workspace_bytes(T, H, I, E, K, moe.FLAG_FORCE_GROUPED)
    atomic_ws = moe.moe_workspace_bytes(T, H, I, E, K,
                                        moe.FLAG_FORCE_GROUPED | moe.FLAG_ATOMIC_COMBINE)
    # the slot path holds two fp32 slot buffers: the split is taken
    assert slot_ws - atomic_ws >= 2 * n * H * 4
    d = cpu_inputs(T, H, I, E, K, seed=135)
    dd = to_device(d)
    rows = np.arange(T)
    assert not y_bf16_for(d, PATHS["slot"])  # a split keeps fp32 partial rows
    a = _run(dd, PATHS["slot"])
    assert_close(a, oracle_rows(d, rows), tight_rows(d, rows, PATHS["slot"]),
                 f"split T={T} I={I}")
    b = _run(dd, PATHS["slot"])
    assert np.array_equal(a, b)
    perm = torch.from_numpy(np.random.default_rng(5).permutation(T))
    pd = dict(dd)
    for k in ("hidden_states", "topk_weights", "topk_ids"):
        pd[k] = dd[k][perm.cuda()].contiguous()
    c = _run(pd, PATHS["slot"])
    assert np.array_equal(c, a[perm.numpy()])
    # the atomic path (no split) stays within the bar of the split path
    e = _run(dd, PATHS["atomic"])
    assert rel_l2(e, a) <= REL_L2_BF16_INTER


@pytest.mark.parametrize("T,H,I,E,K", [
    (4195, 2048, 2048, 8, 2),  # prefill: 384 tiles of 192x256 on 256 CUs
    (8179, 4096, 4096, 8, 2),  # 256x256 tiles, ~4.2 rounds
])
def test_down_projection_tail_split(T, H, I, E, K):
    """Down-projection tiles whose last round would leave at least half the
    chip idle: that round runs as column halves in a second launch. Each
    output element still sums its whole contraction in the same order, so
    every combine path gives the same bits as the single launch
    (MOE_FLAG_NO_TAIL_SPLIT); against the oracle on 256 seeded rows."""
    require_gpu()
    fl = PATHS["slot"]
    assert moe.moe_down_tail_split(T, H, I, E, K, fl)
    assert not moe.moe_down_tail_split(T, H, I, E, K, fl | moe.FLAG_NO_TAIL_SPLIT)
    d = cpu_inputs(T, H, I, E, K, seed=T)
    dd = to_device(d)
    rows = sample_rows(T, 256, seed=2)
    for path, f in (("bf16_y", fl), ("fp32_y", fl | moe.FLAG_FP32_Y), ("atomic", PATHS["atomic"])):
        say(f"tail split T={T} H={H} I={I} E={E} {path}")
        a = _run(dd, f)
        b = _run(dd, f | moe.FLAG_NO_TAIL_SPLIT)
        assert np.array_equal(a, b), path
        if path == "bf16_y":
            assert_close(a[rows], oracle_rows(d, rows), tight_rows(d, rows, f), f"tail T={T}")


def _ids_with_counts(counts, T, K, seed):
    """topk_ids whose expert e holds exactly counts[e] of the T*K slots, every
    token on K distinct experts: the sorted slot list read with stride T (no
    expert holds more than T slots), tokens shuffled."""
    seq = np.repeat(np.arange(len(counts)), counts)
    assert seq.size == T * K and max(counts) <= T
    ids = seq.reshape(K, T).T
    return ids[np.random.default_rng(seed).permutation(T)].astype(np.int32)


@pytest.mark.parametrize("row_tiles", [44, 48, 49, 51])
def test_down_tail_split_set_routings(row_tiles):
    """Prefill's shape (192-row tiles, 8 column tiles of the down projection,
    a round = 32 row tiles) with routings of set expert sizes: 44 row tiles
    leave 3/8 of a round (halves), 48 exactly half (the halves fill one
    round), 49 and 51 leave more than half, where the host's plan still
    splits but the first launch runs every tile and the second finds none.
    Same bits as the single launch on the slot and atomic paths; against the
    oracle on 128 seeded rows."""
    require_gpu()
    T, H, I, E, K = 4195, 2048, 2048, 8, 2
    fl = PATHS["slot"]
    assert moe.moe_down_tail_split(T, H, I, E, K, fl)
    assert moe.moe_m_tile(T, H, I, E, K) == 192
    counts = {44: [1152] * 7 + [326],               # 7*6 + 2
              48: [1049] * 6 + [1048] * 2,          # 8*6, balanced
              49: [1153] + [1034] * 6 + [1033],     # 7 + 7*6
              51: [1153] * 3 + [987] + [986] * 4}[row_tiles]  # 3*7 + 5*6
    assert sum(counts) == T * K and sum(-(-c // 192) for c in counts) == row_tiles
    d = dict(cpu_inputs(T, H, I, E, K, seed=T))
    d["topk_ids"] = torch.from_numpy(_ids_with_counts(counts, T, K, seed=row_tiles))
    dd = to_device(d)
    rows = sample_rows(T, 128, seed=3)
    for path, f in (("slot", fl), ("atomic", PATHS["atomic"])):
        say(f"down tail split, {row_tiles} row tiles, {path}")
        a = _run(dd, f)
        b = _run(dd, f | moe.FLAG_NO_TAIL_SPLIT)
        assert np.array_equal(a, b), path
        if path == "slot":
            assert_close(a[rows], oracle_rows(d, rows), tight_rows(d, rows, f),
                         f"down tail, {row_tiles} row tiles")


@pytest.mark.parametrize("name", ["prefill", "large"])
def test_atomic_path_is_deterministic_for_top2(name):
    """With two routing terms per token the atomic combine is 0 + a + b in
    either order, two-term addition commutes and the hardware atomic add
    rounds to nearest even: run-to-run identical bits, and the same bits as
    the slot path's (0 + a) + b with fp32 slot rows."""
    require_gpu()
    dd = to_device(shape_inputs(name))
    a = _run(dd, PATHS["atomic"])
    b = _run(dd, PATHS["atomic"])
    assert np.array_equal(a, b)
    c = _run(dd, PATHS["slot"] | moe.FLAG_FP32_Y)
    assert np.array_equal(a, c)


@pytest.mark.parametrize("T,H,I,E,K", [
    (1, 128, 128, 1, 1), (37, 128, 256, 4, 4), (129, 256, 128, 16, 1), (1000, 384, 640, 6, 3),
    (3, 512, 256, 8, 2), (20, 128, 128, 128, 8), (300, 256, 384, 64, 6),
])
@pytest.mark.parametrize("path", ["slot", "atomic", "decode", "small_batch"])
def test_ragged_and_degenerate_shapes(T, H, I, E, K, path):
    require_gpu()
    d = cpu_inputs(T, H, I, E, K, seed=T + E)
    dd = to_device(d)
    say(f"shape T={T} H={H} I={I} E={E} K={K} path={path}")
    got = _run(dd, PATHS[path])
    rows = np.arange(T)
    assert_close(got, oracle_rows(d, rows), tight_rows(d, rows, PATHS[path]),
                 f"{T},{H},{I},{E},{K}/{path}")


RANDOM_SHAPES = random_shapes(24, seed=20261203)


@pytest.mark.parametrize("path", ["default", "slot"])
@pytest.mark.parametrize("idx", range(len(RANDOM_SHAPES)))
def test_random_shapes_against_oracle(idx, path):
    require_gpu()
    T, H, I, E, K = RANDOM_SHAPES[idx]
    d = cpu_inputs(T, H, I, E, K, seed=idx)
    dd = to_device(d)
    fl = None if path == "default" else PATHS[path]
    say(f"random shape {idx}: T={T} H={H} I={I} E={E} K={K} path={path} "
        f"(library path {moe.moe_path(T, H, I, E, K, fl or 0)})")
    got = _run(dd, fl)
    rows = sample_rows(T, 48, seed=idx)
    assert_close(got[rows], oracle_rows(d, rows), tight_rows(d, rows, fl),
                 f"random {idx} {T},{H},{I},{E},{K}/{path}")


@pytest.mark.parametrize("T,H,I,E,K", [
    (4195, 2048, 2048, 8, 2),    # 192x256 gate/up; the down projection's column-half tail
    (8192, 4096, 384, 128, 8),   # 256x256 at E=128
    (135, 2048, 2048, 8, 2),     # 64x128 gate/up; contraction split of the down projection
    (520, 4096, 384, 128, 8),    # 64-row tiles
    (1023, 2048, 2048, 8, 2),    # 128x128
    (2400, 2048, 768, 128, 8),   # 192-row tiles at E=128
    (1, 2048, 768, 128, 8),      # per-token path
    (40, 2048, 768, 128, 8),     # per-expert path
])
def test_repeated_calls_are_bitwise_identical(T, H, I, E, K):
    """30 calls in a row into the same output, each compared with the first
    bit for bit: every route is deterministic, so any difference would be a
    race between workgroups or with the workspace."""
    require_gpu()
    dd = to_device(cpu_inputs(T, H, I, E, K, seed=5))
    ref = moe.moe_forward(dd["hidden_states"], dd["w1"], dd["w2"], dd["topk_weights"],
                          dd["topk_ids"], flags=0).clone()
    out = torch.empty_like(ref)
    say(f"repeated calls T={T} H={H} I={I} E={E} K={K} path {moe.moe_path(T, H, I, E, K, 0)}")
    for r in range(30):
        moe.moe_forward(dd["hidden_states"], dd["w1"], dd["w2"], dd["topk_weights"],
                        dd["topk_ids"], out=out, flags=0)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"call {r} differs"


def test_all_tokens_one_expert_and_empty_experts():
    require_gpu()
    d = dict(cpu_inputs(700, 256, 256, 16, 2, seed=5))
    ids = d["topk_ids"].clone()
    ids[:, 0] = 3
    ids[:, 1] = torch.where(ids[:, 1] == 3, torch.full_like(ids[:, 1], 9), ids[:, 1]) % 4 + 8
    d["topk_ids"] = ids.contiguous()
    dd = to_device(d)
    rows = np.arange(700)
    want = oracle_rows(d, rows)
    for path in ("slot", "atomic", "small_batch"):
        assert_close(_run(dd, PATHS[path]), want, tight_rows(d, rows, PATHS[path]),
                     f"one-expert/{path}")


@pytest.mark.parametrize("T,H,I,E,K,skew", [
    (2000, 1024, 1024, 64, 2, "two_hot"),   # 90 % of the slots on experts 0 and 1
    (5000, 2048, 1024, 32, 4, "same_four"),  # every token on experts 0..3
    (1500, 512, 512, 128, 8, "zipf"),        # expert e drawn with weight 1 / (e + 1)
])
def test_skewed_routing_live_tiles(T, H, I, E, K, skew):
    """The grouped GEMMs size their grid for every row tile the routing could
    produce and number only the live ones: with skewed routings (few live
    tiles against that bound, partial tile windows) every tile is computed
    exactly once on the slot and atomic paths (a tile taken twice would be
    added twice on the atomic path)."""
    require_gpu()
    d = dict(cpu_inputs(T, H, I, E, K, seed=T + K))
    rng = np.random.default_rng(T)
    if skew == "two_hot":
        ids = np.stack([rng.permutation(E)[:K] for _ in range(T)])
        hot = rng.random(T) < 0.9
        ids[hot] = np.array([0, 1])
    elif skew == "same_four":
        ids = np.tile(np.arange(K), (T, 1))
    else:
        p = 1.0 / np.arange(1, E + 1)
        ids = np.stack([rng.choice(E, size=K, replace=False, p=p / p.sum()) for _ in range(T)])
    d["topk_ids"] = torch.from_numpy(ids.astype(np.int32))
    dd = to_device(d)
    rows = sample_rows(T, 256, seed=4)
    want = oracle_rows(d, rows)
    for path in ("slot", "atomic"):
        for extra in (0, moe.FLAG_NO_TAIL_SPLIT):
            say(f"skewed {skew} T={T} E={E} K={K} {path} extra={extra}")
            got = _run(dd, PATHS[path] | extra)
            assert_close(got[rows], want, tight_rows(d, rows, PATHS[path]),
                         f"skewed-{skew}/{path}")


def test_out_of_range_ids_are_dropped():
    require_gpu()
    d = dict(cpu_inputs(64, 512, 256, 8, 2, seed=6))
    ids = d["topk_ids"].clone()
    ids[5, 1] = -1
    ids[9, 0] = 8
    zeroed = d["topk_weights"].clone()
    zeroed[5, 1] = 0
    zeroed[9, 0] = 0
    bad = dict(d, topk_ids=ids)
    ref = dict(d, topk_weights=zeroed)
    rows = np.arange(64)
    want = oracle_rows(ref, rows)
    for path in ("slot", "atomic", "decode", "small_batch"):
        got = _run(to_device(bad), PATHS[path])
        assert_close(got, want, None, f"dropped-ids/{path}")


def test_validate_flag_reports_bad_ids():
    require_gpu()
    d = dict(cpu_inputs(64, 512, 256, 8, 2, seed=6))
    good = to_device(d)
    moe.moe_forward(**{k: good[k] for k in ("hidden_states", "w1", "w2", "topk_weights",
                                             "topk_ids")}, flags=moe.FLAG_VALIDATE_IDS)
    for mutate in ("range", "duplicate"):
        ids = d["topk_ids"].clone()
        if mutate == "range":
            ids[10, 1] = 99
        else:
            ids[10, 1] = ids[10, 0]
        bad = dict(good, topk_ids=ids.cuda())
        with pytest.raises(moe.MoeError) as ei:
            moe.moe_forward(**{k: bad[k] for k in ("hidden_states", "w1", "w2", "topk_weights",
                                                    "topk_ids")}, flags=moe.FLAG_VALIDATE_IDS)
        assert ei.value.code == moe.MOE_ERR_INVALID_ARG


def test_zero_tokens_and_errors():
    require_gpu()
    d = to_device(cpu_inputs(4, 128, 128, 4, 2))
    empty = {k: v[:0] for k, v in d.items()}
    out = moe.moe_forward(empty["hidden_states"], d["w1"], d["w2"], empty["topk_weights"],
                          empty["topk_ids"])
    assert out.shape == (0, 128)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_forward(d["hidden_states"], d["w1"], d["w2"], d["topk_weights"], d["topk_ids"],
                        flags=0, workspace=torch.empty(16, dtype=torch.uint8, device="cuda"))
    assert ei.value.code == moe.MOE_ERR_WORKSPACE


def test_caller_workspace_and_side_stream():
    require_gpu()
    s = SHAPES["tiny"]
    d = shape_inputs("tiny")
    dd = to_device(d)
    ref = _run(dd, PATHS["slot"])
    nbytes = moe.moe_workspace_bytes(s.T, s.H, s.I, s.E, s.K, PATHS["slot"])
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        out = moe.moe_forward(dd["hidden_states"], dd["w1"], dd["w2"], dd["topk_weights"],
                              dd["topk_ids"], flags=PATHS["slot"], workspace=ws)
    side.synchronize()
    assert np.array_equal(out.cpu().numpy(), ref)


def test_decode_path_with_caller_workspace_of_garbage():
    """The decode path with a caller workspace full of arbitrary bytes gives
    the internal-workspace result, twice in a row (the per-token kernels
    write every activation value they read back)."""
    require_gpu()
    s = SHAPES["decode"]
    dd = to_device(shape_inputs("decode"))
    fl = moe.FLAG_FORCE_DECODE
    ref = _run(dd, fl)
    nbytes = moe.moe_workspace_bytes(s.T, s.H, s.I, s.E, s.K, fl)
    ws = torch.full((nbytes,), 0xA5, dtype=torch.uint8, device="cuda")
    for _ in range(2):
        out = moe.moe_forward(dd["hidden_states"], dd["w1"], dd["w2"], dd["topk_weights"],
                              dd["topk_ids"], flags=fl, workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), ref)


def test_decode_after_grouped_calls_and_back_to_back():
    """Grouped calls between decode calls share the internal workspace; 40
    decode calls queued without a host sync all give the same bits; so does
    the debug-sync flag."""
    require_gpu()
    dd = to_device(shape_inputs("decode"))
    tiny = to_device(shape_inputs("tiny"))
    ref = _run(dd, None)
    _run(tiny, PATHS["slot"])
    assert np.array_equal(_run(dd, None), ref)
    outs = [moe.moe_forward(dd["hidden_states"], dd["w1"], dd["w2"], dd["topk_weights"],
                            dd["topk_ids"]) for _ in range(40)]
    torch.cuda.synchronize()
    for o in outs:
        assert np.array_equal(o.cpu().numpy(), ref)
    assert np.array_equal(_run(dd, moe.FLAG_DEBUG_SYNC), ref)


@pytest.mark.parametrize("shape", [(2048, 768, 128, 8), (2048, 2048, 8, 2), (512, 256, 8, 2)])
def test_decode_tokens_are_independent(shape):
    """On the decode path each output row depends on its own token only: token
    0 gives the same bits alone and beside a second token, and both rows
    match the oracle."""
    require_gpu()
    H, I, E, K = shape
    d = cpu_inputs(2, H, I, E, K, seed=11)
    dd = to_device(d)
    fl = moe.FLAG_FORCE_DECODE
    two = _run(dd, fl)
    one = _run({k: (v[:1] if k in ("hidden_states", "topk_weights", "topk_ids") else v)
                for k, v in dd.items()}, fl)
    assert np.array_equal(one[0], two[0])
    rows = np.arange(2)
    assert_close(two, oracle_rows(d, rows), tight_rows(d, rows, fl),
                 f"decode-two-tokens/{shape}")


@pytest.mark.parametrize("name,path", [
    ("tiny", "slot"), ("prefill", "slot"), ("prefill", "atomic"), ("decode", "decode"),
    ("tiny", "small_batch"),
])
def test_debug_sync_flag(name, path):
    """MOE_FLAG_DEBUG_SYNC (a synchronisation and a check of the workspace
    guard bands after every stage) leaves the results' bits unchanged, and no
    stage writes past its workspace region on any path (prefill takes the
    down projection's tail launch)."""
    require_gpu()
    dd = to_device(shape_inputs(name))
    say(f"debug sync {name} {path}")
    a = _run(dd, PATHS[path] | moe.FLAG_DEBUG_SYNC)
    b = _run(dd, PATHS[path])
    assert np.array_equal(a, b)


def test_largest_shapes_row():
    """The largest row of the shapes table (T=45936, H=2048, I=768, E=128,
    top-8): full-size run, 1024 seeded rows (first and last included)
    against the oracle."""
    require_gpu()
    T, H, I, E, K = 45936, 2048, 768, 128, 8
    d = cpu_inputs(T, H, I, E, K, seed=0)
    dd = to_device(d)
    say("forward largest shapes-table row")
    got = _run(dd, None)
    rows = sample_rows(T, 1024, seed=5)
    assert_close(got[rows], oracle_rows(d, rows), tight_rows(d, rows, None),
                 "shapes-row-14")


def test_single_hip_runtime_is_mapped():
    """torch and the library share one HIP runtime (stream handles are valid)."""
    require_gpu()
    moe.load_library()
    maps = open("/proc/self/maps").read()
    libs = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    assert len(libs) == 1, libs
    assert any("libmoe_topk_ids.so" in line for line in maps.splitlines())


@pytest.mark.parametrize("T,H,I,E,K", [
    (64, 128, 128, 1024, 8),    # the largest expert count
    (33, 128, 256, 1, 1),       # one expert, top-1
    (5, 8192, 128, 16, 4),      # the largest hidden size the per-token path holds
    (3, 256, 8192, 8, 2),       # a wide intermediate on every path
])
@pytest.mark.parametrize("path", ["default", "slot", "atomic", "decode", "small_batch"])
def test_extreme_sizes(T, H, I, E, K, path):
    require_gpu()
    d = cpu_inputs(T, H, I, E, K, seed=T + H)
    dd = to_device(d)
    say(f"extreme T={T} H={H} I={I} E={E} K={K} path={path}")
    fl = None if path == "default" else PATHS[path]
    got = _run(dd, fl)
    rows = np.arange(T)
    assert_close(got, oracle_rows(d, rows), tight_rows(d, rows, fl),
                 f"extreme {T},{H},{I},{E},{K}/{path}")


def test_binding_rejects_bad_tensors():
    require_gpu()
    dd = to_device(shape_inputs("tiny"))
    with pytest.raises(ValueError):  # not contiguous
        moe.moe_forward(dd["hidden_states"].t().contiguous().t(), dd["w1"], dd["w2"],
                        dd["topk_weights"], dd["topk_ids"])
    with pytest.raises(ValueError):  # wrong dtype
        moe.moe_forward(dd["hidden_states"].float(), dd["w1"], dd["w2"], dd["topk_weights"],
                        dd["topk_ids"])
    with pytest.raises(ValueError):  # host tensor
        moe.moe_forward(dd["hidden_states"].cpu(), dd["w1"], dd["w2"], dd["topk_weights"],
                        dd["topk_ids"])
    with pytest.raises(ValueError):  # inconsistent shapes
        moe.moe_forward(dd["hidden_states"], dd["w1"], dd["w2"][:, :, :-128].contiguous(),
                        dd["topk_weights"], dd["topk_ids"])
    with pytest.raises(ValueError):  # unknown activation
        moe.moe_forward(dd["hidden_states"], dd["w1"], dd["w2"], dd["topk_weights"],
                        dd["topk_ids"], activation="relu")


@pytest.mark.parametrize("name", ["prefill", "wide"])
def test_bf16_expert_outputs_against_fp32_rows(name):
    """The slot path with bf16 expert outputs against the same path with fp32
    ones: every output within sum_k |w_k| * |y_k| * 2^-8 (half a bf16 ulp per
    term) of the fp32 one, where y_k comes from the fp32-row run of a single
    slot; both bitwise run-to-run stable."""
    require_gpu()
    s = SHAPES[name]
    d = shape_inputs(name)
    dd = to_device(d)
    fl16 = PATHS["slot"] | moe.FLAG_BF16_Y
    fl32 = PATHS["slot"] | moe.FLAG_FP32_Y
    a16, a32 = _run(dd, fl16), _run(dd, fl32)
    assert np.array_equal(a16, _run(dd, fl16))
    bound = np.zeros((s.T, s.H))
    for k in range(s.K):  # |y_k|: one slot per token, weight 1, fp32 rows
        one = dict(dd, topk_ids=dd["topk_ids"][:, k:k + 1].contiguous(),
                   topk_weights=torch.ones((s.T, 1), dtype=torch.float32, device="cuda"))
        yk = _run(one, fl32)
        bound += np.abs(d["topk_weights"].numpy()[:, k:k + 1]) * np.abs(yk) * 2.0 ** -8 * 1.001
    diff = np.abs(a16.astype(np.float64) - a32)
    slack = 1e-6 * np.max(np.abs(a32))
    say(f"bf16 vs fp32 expert outputs {name}: max diff {diff.max():.3e}, "
        f"max diff / bound {np.max(diff / (bound + slack)):.3f}, "
        f"differing {np.mean(a16 != a32):.3f}")
    assert np.all(diff <= bound + slack)


def test_bf16_expert_outputs_forced_on_a_split_shape():
    """T=135, H=I=2048, E=8, top-2 splits the down projection with fp32 rows;
    asking for bf16 rows drops the split and matches the oracle's bf16-output
    mode on every row."""
    require_gpu()
    T, H, I, E, K = 135, 2048, 2048, 8, 2
    d = cpu_inputs(T, H, I, E, K, seed=135)
    dd = to_device(d)
    fl = PATHS["slot"] | moe.FLAG_BF16_Y
    assert y_bf16_for(d, fl) and not y_bf16_for(d, PATHS["slot"])
    rows = np.arange(T)
    assert_close(_run(dd, fl), oracle_rows(d, rows), tight_rows(d, rows, fl), "split+bf16 rows")
