"""CPU-side checks of the C ABI: the library loads, exports every function the
header declares, and rejects bad arguments before touching a device."""
import ctypes
import os
import re

import pytest

import moe_topk_ids_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_topk_ids.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)
    return sorted({n for n in names if n.startswith("moe_")})


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(moe.LIB_PATH):
        pytest.fail("libmoe_topk_ids.so is not built (python -m moe_topk_ids_amd.build)")
    return moe.load_library()


def test_header_declares_the_api():
    names = _declared_functions()
    for n in ("moe_forward", "moe_forward_ex", "moe_workspace_bytes", "moe_m_tile", "moe_route",
              "moe_route_scratch_bytes", "moe_gemm1_silu", "moe_last_error", "moe_release",
              "moe_uses_decode_path", "moe_topk_softmax", "moe_path", "moe_forward_act", "moe_forward_fp8",
              "moe_gemm1_silu_fp8", "moe_fp8_widens_in_gemm", "moe_forward_noalloc"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for n in _declared_functions():
        assert hasattr(lib, n), f"symbol {n} missing"


def test_size_validation_without_device(lib):
    p = ctypes.c_void_p(0)
    # K > E
    rc = lib.moe_forward_ex(p, p, p, p, p, 4, 128, 128, 2, 3, p, 0, p, 0, p)
    assert rc == moe.MOE_ERR_INVALID_ARG
    assert b"top_k" in lib.moe_last_error()
    # H not a multiple of 128
    rc = lib.moe_forward_ex(p, p, p, p, p, 4, 100, 128, 8, 2, p, 0, p, 0, p)
    assert rc == moe.MOE_ERR_UNSUPPORTED
    # negative T
    rc = lib.moe_forward_ex(p, p, p, p, p, -1, 128, 128, 8, 2, p, 0, p, 0, p)
    assert rc == moe.MOE_ERR_INVALID_ARG
    # too many experts
    rc = lib.moe_forward_ex(p, p, p, p, p, 4, 128, 128, 2048, 2, p, 0, p, 0, p)
    assert rc == moe.MOE_ERR_UNSUPPORTED
    # null pointers with T > 0
    rc = lib.moe_forward(p, p, p, p, p, 4, 128, 128, 8, 2, p, p)
    assert rc == moe.MOE_ERR_INVALID_ARG
    # T == 0 is a no-op success even with null pointers
    assert lib.moe_forward(p, p, p, p, p, 0, 128, 128, 8, 2, p, p) == moe.MOE_OK


def test_activation_argument_validation(lib):
    p = ctypes.c_void_p(0)
    f = ctypes.c_float
    # unknown activation; swigluoai with a negative limit
    assert lib.moe_forward_act(p, p, p, p, p, 4, 128, 128, 8, 2, 7, f(1.0), f(7.0), p, p, p, 0, p,
                               0, p) == moe.MOE_ERR_INVALID_ARG
    assert b"activation" in lib.moe_last_error()
    assert lib.moe_forward_act(p, p, p, p, p, 4, 128, 128, 8, 2, moe.ACT_SWIGLUOAI, f(1.0),
                               f(-1.0), p, p, p, 0, p, 0, p) == moe.MOE_ERR_INVALID_ARG
    # T == 0 is a no-op for every activation
    for a in range(4):
        assert lib.moe_forward_act(p, p, p, p, p, 0, 128, 128, 8, 2, a, f(1.702), f(7.0), p, p, p,
                                   0, p, 0, p) == moe.MOE_OK


def test_fp8_argument_validation(lib):
    p = ctypes.c_void_p(0)
    f = ctypes.c_float
    # a scale block that is not a multiple of 128, or does not divide I
    for block in (64, 200, 256):
        rc = lib.moe_forward_fp8(p, p, p, p, p, block, p, p, 4, 512, 384, 8, 2, 0, f(1.702), f(7.0),
                                 p, p, p, 0, p, 0, p)
        assert rc == moe.MOE_ERR_UNSUPPORTED, block
    # null weights with T > 0
    assert lib.moe_forward_fp8(p, p, p, p, p, 128, p, p, 4, 512, 384, 8, 2, 0, f(1.702), f(7.0),
                               p, p, p, 0, p, 0, p) == moe.MOE_ERR_INVALID_ARG
    # grouped path: with many experts and few rows each the GEMMs widen FP8
    # fragments in registers (no extra workspace); for dense experts, or when
    # H/128 or I/128 exceeds 32 (the tile's scales no longer fit in LDS), a
    # pass first widens the weights into a bf16 copy in the workspace
    fl = moe.FLAG_FORCE_GROUPED

    def extra(*shape):
        return (moe.moe_workspace_bytes(*shape, fl | moe.FLAG_FP8_WEIGHTS)
                - moe.moe_workspace_bytes(*shape, fl))
    assert extra(8192, 4096, 384, 128, 8) == 0
    assert extra(4195, 2048, 2048, 8, 2) >= 8 * 3 * 2048 * 2048 * 2
    assert extra(100, 4224, 512, 8, 2) >= 8 * 3 * 4224 * 512 * 2
    assert moe.moe_path(1, 2048, 768, 128, 8, moe.FLAG_FP8_WEIGHTS) == moe.PATH_DECODE
    # which widening the grouped path takes
    assert moe.moe_fp8_widens_in_gemm(8192, 4096, 384, 128, 8, 128)      # many experts, few rows
    assert not moe.moe_fp8_widens_in_gemm(4195, 2048, 2048, 8, 2, 256)  # dense experts
    assert not moe.moe_fp8_widens_in_gemm(100, 4224, 512, 8, 2, 128)    # 33 scale blocks per row
    assert lib.moe_fp8_widens_in_gemm(4, 512, 384, 8, 2, 200) == moe.MOE_ERR_UNSUPPORTED
    # the standalone FP8 GEMM1 checks its block before touching a device
    for block, H in ((64, 512), (128, 4224)):
        rc = lib.moe_gemm1_silu_fp8(p, p, p, block, p, p, p, 4, H, 384, 8, 2, 128, 1, p, p)
        assert rc == moe.MOE_ERR_UNSUPPORTED, (block, H)


def test_route_argument_validation(lib):
    p = ctypes.c_void_p(0)
    # m_tile must be a multiple of 16 in [16, 256]
    for m in (8, 40, 272):
        assert lib.moe_route(p, 4, 2, 8, m, p, p, p, p, p, p, 1000, p, p) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_route(p, 4, 2, 8, 64, p, p, p, p, p, p, 10, p, p) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_gemm1_silu(p, p, p, p, p, 4, 128, 128, 8, 2, 32, 1, p, p) == moe.MOE_ERR_UNSUPPORTED


def test_router_argument_validation(lib):
    p = ctypes.c_void_p(0)
    assert lib.moe_topk_softmax(p, 4, 8, 9, 1, p, p, p) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_topk_softmax(p, 4, 2000, 2, 1, p, p, p) == moe.MOE_ERR_UNSUPPORTED
    assert lib.moe_topk_softmax(p, 4, 64, 40, 1, p, p, p) == moe.MOE_ERR_UNSUPPORTED
    assert lib.moe_topk_softmax(p, 0, 8, 2, 1, p, p, p) == moe.MOE_OK
    assert lib.moe_topk_softmax(p, 3, 8, 2, 1, p, p, p) == moe.MOE_ERR_INVALID_ARG


def test_workspace_and_tile_queries(lib):
    assert moe.moe_workspace_bytes(0, 512, 256, 8, 2) == 0
    ws_slot = moe.moe_workspace_bytes(4195, 2048, 2048, 8, 2)
    ws_fp32 = moe.moe_workspace_bytes(4195, 2048, 2048, 8, 2, moe.FLAG_FP32_Y)
    ws_atomic = moe.moe_workspace_bytes(4195, 2048, 2048, 8, 2, moe.FLAG_ATOMIC_COMBINE)
    # the slot path holds the per-slot outputs [T*K, H]: bf16 by default
    # here, fp32 with the flag; the atomic path none
    assert moe.moe_y_bf16(4195, 2048, 2048, 8, 2)
    assert not moe.moe_y_bf16(4195, 2048, 2048, 8, 2, moe.FLAG_FP32_Y)
    assert not moe.moe_y_bf16(4195, 2048, 2048, 8, 2, moe.FLAG_ATOMIC_COMBINE)
    assert ws_slot - ws_atomic >= 4195 * 2 * 2048 * 2
    assert ws_fp32 - ws_atomic >= 4195 * 2 * 2048 * 4
    # the split down projection of few-token E=8 rows keeps fp32 partial rows,
    # unless bf16 rows are asked for (then no split)
    assert not moe.moe_y_bf16(135, 2048, 2048, 8, 2)
    assert moe.moe_y_bf16(135, 2048, 2048, 8, 2, moe.FLAG_BF16_Y)
    assert (moe.moe_workspace_bytes(135, 2048, 2048, 8, 2)
            > moe.moe_workspace_bytes(135, 2048, 2048, 8, 2, moe.FLAG_BF16_Y))
    # the streaming paths keep fp32
    assert not moe.moe_y_bf16(1, 2048, 768, 128, 8)
    assert moe.moe_m_tile(4195, 2048, 2048, 8, 2) in (64, 128, 192, 256)
    assert moe.moe_uses_decode_path(1, 2048, 768, 128, 8)
    assert not moe.moe_uses_decode_path(4195, 2048, 2048, 8, 2)
    assert moe.moe_uses_decode_path(4195, 2048, 2048, 8, 2, moe.FLAG_FORCE_DECODE)
    assert not moe.moe_uses_decode_path(1, 2048, 768, 128, 8, moe.FLAG_FORCE_GROUPED)
    with pytest.raises(moe.MoeError):
        moe.moe_m_tile(1, 100, 128, 8, 2)


def test_tile_choice(lib):
    # the cost model's picks on shapes where the measured winner is clear
    # ~34 rows per expert: 64-row tiles, 64x128 for the gate/up product (three
    # workgroups per CU, all tiles in one round)
    assert moe.moe_m_tile(135, 2048, 2048, 8, 2) == 64
    assert moe.moe_m_tile(277, 2048, 2048, 8, 2) == 128    # ~69 rows: one 128-row tile each
    assert moe.moe_m_tile(668, 2048, 2048, 8, 2) == 64     # ~167 rows per expert: least padding
    assert moe.moe_m_tile(8192, 4096, 384, 128, 8) == 256  # many tiles: the big tile's efficiency
    assert moe.moe_m_tile(15381, 4096, 4096, 8, 2) == 256
    # ~1050 rows per expert: 192-row tiles pad like 128-row ones (256-row
    # tiles pad to 1280) and make exactly three rounds; measured fastest
    assert moe.moe_m_tile(4195, 2048, 2048, 8, 2) == 192
    assert moe.moe_m_tile(4098, 4096, 4096, 8, 2) == 192
    assert moe.moe_m_tile(2400, 2048, 768, 128, 8) == 192  # ~150 rows per expert: one tile each


def test_path_choice(lib):
    assert moe.moe_path(1, 2048, 768, 128, 8) == moe.PATH_DECODE
    assert moe.moe_path(4195, 2048, 2048, 8, 2) == moe.PATH_GROUPED
    fl = moe.FLAG_FORCE_SMALL_BATCH
    assert moe.moe_path(100, 2048, 2048, 8, 2, fl) == moe.PATH_SMALL_BATCH
    # past the small-batch slot limit the forced path falls back to grouped
    assert moe.moe_path(600, 2048, 2048, 8, 2, fl) == moe.PATH_GROUPED
    assert moe.moe_path(1, 2048, 768, 128, 8, moe.FLAG_FORCE_GROUPED) == moe.PATH_GROUPED
    # default choice by size (the measured crossovers)
    assert moe.moe_path(8, 2048, 768, 128, 8) == moe.PATH_DECODE
    assert moe.moe_path(32, 2048, 768, 128, 8) == moe.PATH_SMALL_BATCH
    assert moe.moe_path(128, 2048, 768, 128, 8) == moe.PATH_GROUPED
    assert moe.moe_path(2, 2048, 2048, 8, 2) == moe.PATH_DECODE
    assert moe.moe_path(16, 2048, 2048, 8, 2) == moe.PATH_SMALL_BATCH
    assert moe.moe_path(135, 2048, 2048, 8, 2) == moe.PATH_GROUPED
    # the small-batch / grouped crossovers of the sweep the path model was fitted to
    # (each side the faster path measured there)
    assert moe.moe_path(24, 2048, 2048, 8, 2) == moe.PATH_SMALL_BATCH
    assert moe.moe_path(32, 2048, 2048, 8, 2) == moe.PATH_GROUPED
    assert moe.moe_path(48, 2048, 768, 128, 8) == moe.PATH_SMALL_BATCH
    assert moe.moe_path(64, 2048, 768, 128, 8) == moe.PATH_GROUPED
    assert moe.moe_path(64, 4096, 384, 128, 8) == moe.PATH_GROUPED
    assert moe.moe_path(16, 4096, 4096, 8, 2) == moe.PATH_SMALL_BATCH
    assert moe.moe_path(24, 4096, 4096, 8, 2) == moe.PATH_GROUPED
    assert moe.moe_uses_decode_path(8, 2048, 768, 128, 8)
    assert not moe.moe_uses_decode_path(32, 2048, 768, 128, 8)
    # the small-batch workspace holds the bf16 activations and fp32 slot rows
    ws = moe.moe_workspace_bytes(100, 2048, 2048, 8, 2, fl)
    assert ws >= 200 * 2048 * 2 + 200 * 2048 * 4


def test_noalloc_rejects_sizes_beyond_its_array_on_the_host(lib):
    """moe_forward_noalloc checks its workspace need against the static
    array before any device call: the large workload is refused with a
    message naming both sizes; invalid sizes still get the size errors."""
    p = ctypes.c_void_p(0)
    rc = lib.moe_forward_noalloc(p, p, p, p, p, 15381, 4096, 4096, 8, 2, p, 0, p)
    assert rc == moe.MOE_ERR_WORKSPACE
    msg = lib.moe_last_error().decode()
    assert "static scratch" in msg and str(moe.NOALLOC_SCRATCH_BYTES) in msg
    assert str(lib.moe_workspace_bytes(15381, 4096, 4096, 8, 2, 0)) in msg
    assert lib.moe_forward_noalloc(p, p, p, p, p, 4, 128, 128, 2, 3, p, 0, p) == \
        moe.MOE_ERR_INVALID_ARG
    # prefill's workspace fits the array
    assert 0 < lib.moe_workspace_bytes(4195, 2048, 2048, 8, 2, 0) <= moe.NOALLOC_SCRATCH_BYTES


def test_workspace_limit_gives_alloc_error_before_any_device_work():
    """MOE_WORKSPACE_LIMIT caps the internal workspace: a call that would need
    more returns MOE_ERR_ALLOC, and does so before any HIP call (this runs
    without a GPU); a call with its own workspace is not limited (it then
    reaches the device and fails differently here)."""
    import subprocess
    import sys
    code = (
        "import ctypes, moe_topk_ids_amd as moe\n"
        "lib = moe.load_library()\n"
        "p = ctypes.c_void_p(256)\n"
        "rc = lib.moe_forward_ex(p, p, p, p, p, 4195, 2048, 2048, 8, 2, p, 0, None, 0, None)\n"
        "print(rc, lib.moe_last_error().decode())\n"
        "need = lib.moe_workspace_bytes(4195, 2048, 2048, 8, 2, 0)\n"
        "rc2 = lib.moe_forward_ex(p, p, p, p, p, 4195, 2048, 2048, 8, 2, p, 0, p, need, None)\n"
        "print(rc2)\n")
    env = dict(os.environ, MOE_WORKSPACE_LIMIT="4096")
    r = subprocess.run([sys.executable, "-c", code], env=env, cwd=ROOT, capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    first, second = r.stdout.strip().splitlines()[-2:]
    rc, msg = first.split(" ", 1)
    assert int(rc) == moe.MOE_ERR_ALLOC
    assert "MOE_WORKSPACE_LIMIT=4096" in msg
    assert int(second) != moe.MOE_ERR_ALLOC


def test_debug_sync_layout_holds_guard_bands(lib):
    """With MOE_FLAG_DEBUG_SYNC the workspace layout places a 256-byte guard
    band after every region: the size grows by whole bands on every path."""
    for shape, regions in (((4195, 2048, 2048, 8, 2), 10),  # grouped: 10 regions
                           ((1, 2048, 768, 128, 8), 2),     # per token: error flag, act
                           ((40, 2048, 768, 128, 8), 3)):   # small batch: + slot rows
        plain = lib.moe_workspace_bytes(*shape, 0)
        guarded = lib.moe_workspace_bytes(*shape, moe.FLAG_DEBUG_SYNC)
        assert guarded - plain == regions * 256, shape


def test_tail_split_plan(lib):
    """The down projection's column-half tail launch is planned for the prefill
    shape (384 tiles of 192x256: 1.5 rounds) and T=8179, H=I=4096 (~4.2
    rounds), not where its contraction is short (I=384: 6 stages), not with
    FP8 weights, not with MOE_FLAG_NO_TAIL_SPLIT, and not on the streaming
    paths."""
    assert moe.moe_down_tail_split(4195, 2048, 2048, 8, 2, 0)
    assert moe.moe_down_tail_split(8179, 4096, 4096, 8, 2, 0)
    assert not moe.moe_down_tail_split(3936, 4096, 384, 128, 8, 0)
    assert not moe.moe_down_tail_split(4195, 2048, 2048, 8, 2, moe.FLAG_FP8_WEIGHTS)
    assert not moe.moe_down_tail_split(4195, 2048, 2048, 8, 2, moe.FLAG_NO_TAIL_SPLIT)
    assert not moe.moe_down_tail_split(1, 2048, 768, 128, 8, 0)
    assert not moe.moe_down_tail_split(15381, 4096, 4096, 8, 2, 0)  # whole rounds
    assert lib.moe_down_tail_split(4, 100, 128, 8, 2, 0) == moe.MOE_ERR_UNSUPPORTED
