"""Host-side tests of libdgemm (no GPU): the library loads and exports every entry point
of include/dgemm.h, plans validate their arguments, the planner's split-K search and LDS
row permutation agree with the oracle's reading of the pages, and gemm_run rejects bad
arguments before touching the device."""
import ctypes
import os
import re

import numpy as np
import pytest

import dense_gemm_operand_amd as dg
import oracle
from helpers import env

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dgemm.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gemm_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert _declared_functions() == sorted([
        "gemm_plan", "gemm_workspace_size", "gemm_run", "gemm_plan_query",
        "gemm_plan_destroy", "gemm_status_string", "gemm_lds_row_perm", "gemm_pack_u4_tiled",
        "gemm_run_noalloc"])


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(dg.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    for st in range(-6, 1):
        assert dg.gemm_status_string(st) not in ("", "unknown status")
    assert dg.gemm_status_string(-99) == "unknown status"


def _plan_status(*args, quant=None):
    h = ctypes.c_void_p()
    q = ctypes.byref(quant) if quant is not None else None
    st = dg.lib().gemm_plan(ctypes.byref(h), *args, q)
    if h.value:
        dg.gemm_plan_destroy(h.value)
    return st, h.value


F16, BF16, U4, F32 = dg.GEMM_F16, dg.GEMM_BF16, dg.GEMM_U4, dg.GEMM_F32
ROW, COL = dg.GEMM_ROW_MAJOR, dg.GEMM_COL_MAJOR


@pytest.fixture
def fake_cus():
    with env(DGEMM_FAKE_CU_COUNT=256):
        yield


def test_plan_argument_errors(fake_cus):
    ok = (64, 64, 64, ROW, COL, F16, F16, F16, 0)
    assert _plan_status(*ok)[0] == dg.GEMM_OK
    bad = [
        ((0, 64, 64, ROW, COL, F16, F16, F16, 0), dg.GEMM_ERR_INVALID_ARG),
        ((64, -1, 64, ROW, COL, F16, F16, F16, 0), dg.GEMM_ERR_INVALID_ARG),
        ((64, 64, 64, 2, COL, F16, F16, F16, 0), dg.GEMM_ERR_INVALID_ARG),
        ((64, 64, 64, ROW, COL, 7, F16, F16, 0), dg.GEMM_ERR_INVALID_ARG),
        ((64, 64, 64, ROW, COL, F16, F16, F16, -1), dg.GEMM_ERR_INVALID_ARG),
        ((64, 64, 64, ROW, COL, F16, F16, F16, 3), dg.GEMM_ERR_UNSUPPORTED),
        ((64, 64, 64, ROW, COL, F16, F16, F16, 32), dg.GEMM_ERR_UNSUPPORTED),
        ((64, 64, 64, ROW, COL, F16, BF16, F16, 0), dg.GEMM_ERR_UNSUPPORTED),   # mixed
        ((64, 64, 64, ROW, COL, F32, F32, F32, 0), dg.GEMM_ERR_UNSUPPORTED),    # fp32 in
        ((64, 64, 60, ROW, COL, F16, F16, F16, 0), dg.GEMM_ERR_UNSUPPORTED),    # K % 8
        ((60, 64, 64, COL, COL, F16, F16, F16, 0), dg.GEMM_ERR_UNSUPPORTED),    # M % 8, col A
        ((64, 60, 64, ROW, ROW, F16, F16, F16, 0), dg.GEMM_ERR_UNSUPPORTED),    # N % 8, row B
        ((64, 64, 64, ROW, COL, F16, U4, F16, 0), dg.GEMM_ERR_UNSUPPORTED),     # u4 w/o quant
        ((64, 64, 64, ROW, COL, F16, F16, U4, 0), dg.GEMM_ERR_UNSUPPORTED),     # u4 output
    ]
    for args, want in bad:
        assert _plan_status(*args)[0] == want, args
    q = dg.int4_quant()
    assert _plan_status(64, 64, 256, ROW, COL, F16, U4, F16, 0, quant=q)[0] == dg.GEMM_OK
    assert _plan_status(64, 64, 200, ROW, COL, F16, U4, F16, 0, quant=q)[0] == dg.GEMM_ERR_UNSUPPORTED
    assert _plan_status(64, 64, 256, ROW, ROW, F16, U4, F16, 0, quant=q)[0] == dg.GEMM_ERR_UNSUPPORTED
    assert _plan_status(64, 64, 256, ROW, COL, BF16, U4, F16, 0, quant=q)[0] == dg.GEMM_ERR_UNSUPPORTED
    # group sizes: powers of two from 32 to K dividing K; zero points 0..15
    for g, z, want in [(32, 0, dg.GEMM_OK), (64, 15, dg.GEMM_OK), (256, 3, dg.GEMM_OK),
                       (16, 8, dg.GEMM_ERR_UNSUPPORTED), (48, 8, dg.GEMM_ERR_UNSUPPORTED),
                       (512, 8, dg.GEMM_ERR_UNSUPPORTED), (128, 16, dg.GEMM_ERR_UNSUPPORTED),
                       (128, -1, dg.GEMM_ERR_UNSUPPORTED)]:
        q2 = dg.gemm_quant_t(g, z, F16, 0)
        assert _plan_status(64, 64, 256, ROW, COL, F16, U4, F16, 0, quant=q2)[0] == want, (g, z)
    # M <= 16 with non-contiguous extents that are not multiples of 8 stay allowed where
    # the contiguous index is K
    assert _plan_status(3, 5, 64, ROW, COL, F16, F16, F16, 0)[0] == dg.GEMM_OK


def test_plan_extents_whose_byte_counts_overflow_64_bits(fake_cus):
    # byte counts of extents like these wrap around in 64-bit arithmetic; every one must be
    # refused as beyond the 2 GiB operand limit, never planned
    big = [(1 << 40, 64, 1 << 40, F16), (1 << 62, 64, 64, F16), (64, 1 << 62, 64, F16),
           (64, 64, 1 << 62, F16), ((1 << 31) - 8, (1 << 31) - 8, 64, F32),
           ((1 << 32) + 8, 8, 8, F16)]
    for M, N, K, oc in big:
        assert _plan_status(M, N, K, ROW, COL, F16, F16, oc, 0)[0] == dg.GEMM_ERR_UNSUPPORTED, (M, N, K)
    # the limits themselves: an A of 2 GiB is refused, 256 bytes less (K - 8) is planned
    assert _plan_status(16, 8, 1 << 26, ROW, COL, F16, F16, F16, 1)[0] == dg.GEMM_ERR_UNSUPPORTED
    assert _plan_status(16, 8, (1 << 26) - 8, ROW, COL, F16, F16, F16, 1)[0] == dg.GEMM_OK
    # C (fp32) at exactly 2 GiB is refused, one row less is planned
    assert _plan_status(1 << 15, 1 << 14, 64, ROW, COL, F16, F16, F32, 1)[0] == dg.GEMM_ERR_UNSUPPORTED
    assert _plan_status((1 << 15) - 8, 1 << 14, 64, ROW, COL, F16, F16, F32, 1)[0] == dg.GEMM_OK


def test_plan_without_device_is_no_device():
    with env(DGEMM_FAKE_CU_COUNT=None, HIP_VISIBLE_DEVICES=None):
        import torch
        if torch.cuda.is_available():
            pytest.skip("a device is present")
        assert _plan_status(64, 64, 64, ROW, COL, F16, F16, F16, 0)[0] == dg.GEMM_ERR_NO_DEVICE


@pytest.mark.parametrize("M,N,K,la,lb,dt,db", [
    (16, 8192, 28672, ROW, COL, F16, F16),
    (16, 8192, 8192, ROW, COL, F16, U4),
    (16, 1000, 4096, ROW, COL, BF16, BF16),
    (4096, 4096, 4096, COL, COL, F16, F16),
    (3072, 5120, 6144, COL, ROW, BF16, BF16),
    (256, 256, 256, ROW, ROW, F16, F16),
    (100, 3000, 50000, ROW, ROW, F16, F16),
])
def test_split_k_choice_matches_the_page_search(fake_cus, M, N, K, la, lb, dt, db):
    q = dg.int4_quant() if db == U4 else None
    p = dg.gemm_plan(M, N, K, la, lb, dt, db, F16, 0, q)
    info = dg.gemm_plan_query(p)
    dg.gemm_plan_destroy(p)
    step = info["tile_k"] * (info["waves"] if info["kernel"] == 1 else 1)
    assert info["kernel"] == 0 or info["schedule"] == 0   # the skinny kernel has one loop
    want = oracle.splitk_factor(M, N, K, info["tile_m"], info["tile_n"], step,
                                256 * info["slots_per_cu"])
    assert info["split_k"] == want
    tiles = -(-M // info["tile_m"]) * -(-N // info["tile_n"])
    assert info["grid_x"] * info["grid_y"] * info["grid_z"] == tiles * want
    if want > 1:
        assert info["workspace_bytes"] >= dg.COUNTER_BYTES + want * tiles * info["tile_m"] * info["tile_n"] * 4
    else:
        assert info["workspace_bytes"] == 0


def test_requested_split_k_falls_back_past_the_counter_capacity(fake_cus):
    # one 4-byte arrival counter per output tile in the first 64 KiB of the workspace:
    # 16384 tiles keep the requested factor, 16641 tiles (129 x 129) plan without a split
    with env(DGEMM_FORCE_TILE="128x128"):
        for n, want in ((16384, 4), (16512, 1)):
            p = dg.gemm_plan(n, n, 1024, ROW, COL, F16, F16, F16, 4)
            i = dg.gemm_plan_query(p)
            dg.gemm_plan_destroy(p)
            assert (i["tile_m"], i["tile_n"]) == (128, 128)
            assert i["grid_x"] == (n // 128) ** 2
            assert i["split_k"] == want
            assert (i["workspace_bytes"] > 0) == (want > 1)


def test_headline_plans(fake_cus):
    p = dg.gemm_plan(4096, 4096, 4096, COL, COL, F16, F16, F16, 0)
    i = dg.gemm_plan_query(p)
    dg.gemm_plan_destroy(p)
    assert (i["tile_m"], i["tile_n"], i["split_k"], i["grid_x"]) == (256, 256, 1, 256)
    assert (i["perm_block"], i["perm_stride"], i["lds_pad_bytes"]) == (64, 8, 32)
    assert i["direct_lds"] == 2   # B (column-major, K-contiguous) goes straight to LDS
    assert i["schedule"] == 1     # two wave groups in ping-pong
    assert i["lds_bytes"] <= 160 * 1024
    # 3072x5120: the non-power-of-2 192x320 tile (16 x 16 = 256 tiles, one per CU) on the
    # 8-wave ping-pong with 16x16x32 blocks, against 240 tiles of 256x256; both transposed
    # operands straight into LDS in 64-wide K-row segments (B = 64, S = 8, 64 B pad). The
    # same at 2880x5440 (255 tiles against 264 of 256x256, two rounds on 256 CUs), where the
    # split-K search, counting the one empty slot as waste, doubles up to its cap of 16.
    for M, N, grid, sk in ((3072, 5120, 256, 1), (2880, 5440, 255, 16)):
        p = dg.gemm_plan(M, N, 6144, COL, ROW, BF16, BF16, BF16, 0)
        i = dg.gemm_plan_query(p)
        dg.gemm_plan_destroy(p)
        assert (i["tile_m"], i["tile_n"], i["grid_x"], i["waves"]) == (192, 320, grid, 8)
        assert (i["schedule"], i["mfma_m"], i["direct_lds"], i["split_k"]) == (1, 16, 12, sk)
        assert (i["perm_block"], i["perm_stride"], i["lds_pad_bytes"]) == (64, 8, 64)
    # the 4096^3 headline (NN, in-register transpose of A) on 16x16x32 blocks; 32x32x16 on
    # request
    p = dg.gemm_plan(4096, 4096, 4096, COL, COL, F16, F16, F16, 0)
    assert dg.gemm_plan_query(p)["mfma_m"] == 16
    dg.gemm_plan_destroy(p)
    with env(DGEMM_FORCE_MFMA=32):
        p = dg.gemm_plan(4096, 4096, 4096, COL, COL, F16, F16, F16, 0)
        i = dg.gemm_plan_query(p)
        dg.gemm_plan_destroy(p)
    assert (i["mfma_m"], i["schedule"], i["direct_lds"], i["perm_block"]) == (32, 1, 2, 64)


@pytest.mark.parametrize("dt", [F16, BF16])
@pytest.mark.parametrize("M,N,K", [(4096, 4096, 4096), (3072, 5120, 6144), (8192, 8192, 520)])
def test_default_loader_and_schedule_per_layout(fake_cus, dt, M, N, K):
    # every layout runs the 8-wave ping-pong schedule. On 256x256 tiles K-contiguous
    # operands go straight into LDS; NN's transposed A is transposed in registers (64-row
    # stride-8 permuted rows), TT's and NT's transposed operands go straight into LDS in
    # global order, in 64-wide K-row segments (B = 64, S = 8, 64 B pad), and the LDS reads
    # transpose them. At 3072x5120 the 192x320 tile (16x16x32 blocks) takes every
    # operand straight into LDS, transposed ones in the same segments.
    if (M, N) == (3072, 5120):
        tile, mfma = (192, 320), 16
        want = {(ROW, COL): (3, (1, 1), 0), (COL, COL): (6, (64, 8), 64),
                (ROW, ROW): (9, (64, 8), 64), (COL, ROW): (12, (64, 8), 64)}
    else:
        # 16x16x32 blocks in every layout, TT's and NT's transposed operands in 64-wide
        # K-row segments
        tile, mfma = (256, 256), 16
        # (thread-stored transposed rows of the 16x16x32 kernels: 32-byte pad and chunk swap)
        want = {(ROW, COL): (3, (1, 1), 0), (COL, COL): (2, (64, 8), 32),
                (ROW, ROW): (9, (64, 8), 64), (COL, ROW): (12, (64, 8), 64)}
    for (la, lb), (bits, perm, pad) in want.items():
        p = dg.gemm_plan(M, N, K, la, lb, dt, dt, dt, 1)
        i = dg.gemm_plan_query(p)
        dg.gemm_plan_destroy(p)
        assert (i["tile_m"], i["tile_n"], i["waves"], i["schedule"]) == (*tile, 8, 1), (la, lb)
        assert i["mfma_m"] == mfma, (la, lb)
        assert i["direct_lds"] == bits, (la, lb)
        assert (i["perm_block"], i["perm_stride"]) == perm, (la, lb)
        assert i["lds_pad_bytes"] == pad, (la, lb)
        assert i["lds_bytes"] <= 160 * 1024
    # the in-register transpose stays selectable for NT, and for TT's B on 16x16x32 blocks
    with env(DGEMM_FORCE_DTL=0):
        p = dg.gemm_plan(M, N, K, COL, ROW, dt, dt, dt, 1)
        i = dg.gemm_plan_query(p)
        dg.gemm_plan_destroy(p)
    assert (i["direct_lds"], i["schedule"], i["perm_block"]) == (0, 1, 64)
    if tile == (256, 256):
        with env(DGEMM_FORCE_DTL=1, DGEMM_FORCE_MFMA=16):
            p = dg.gemm_plan(M, N, K, ROW, ROW, dt, dt, dt, 1)
            i = dg.gemm_plan_query(p)
            dg.gemm_plan_destroy(p)
        assert (i["direct_lds"], i["mfma_m"], i["perm_block"], i["lds_pad_bytes"]) == (1, 16, 64, 32)


def test_lds_row_permutation_matches_the_page_formula():
    for B in range(1, 257):
        for S in range(1, B + 1):
            if B % S:
                assert dg.gemm_lds_row_perm(B, S, 0, False) == -1
                continue
            f = [dg.gemm_lds_row_perm(B, S, i, False) for i in range(B)]
            assert f == [oracle.perm_fwd(i, B, S) for i in range(B)]
            assert [dg.gemm_lds_row_perm(B, S, x, True) for x in f] == list(range(B))
    assert dg.gemm_lds_row_perm(8, 2, 8, False) == -1


def test_run_rejects_bad_arguments_before_any_device_work(fake_cus):
    p = dg.gemm_plan(128, 128, 4096, ROW, COL, F16, F16, F16, 4)
    try:
        need = dg.gemm_workspace_size(p)
        assert need > 0
        L = dg.lib()
        A, B, C, W = 0x10000, 0x20000, 0x30000, 0x40000   # never dereferenced
        assert L.gemm_run(None, A, B, None, C, W, need, None) == dg.GEMM_ERR_INVALID_ARG
        assert L.gemm_run(p, None, B, None, C, W, need, None) == dg.GEMM_ERR_INVALID_ARG
        assert L.gemm_run(p, A + 8, B, None, C, W, need, None) == dg.GEMM_ERR_MISALIGNED
        assert L.gemm_run(p, A, B, None, C + 2, W, need, None) == dg.GEMM_ERR_MISALIGNED
        assert L.gemm_run(p, A, B, None, C, None, need, None) == dg.GEMM_ERR_INVALID_ARG
        assert L.gemm_run(p, A, B, None, C, W, need - 16, None) == dg.GEMM_ERR_WORKSPACE_TOO_SMALL
        assert L.gemm_run(p, A, B, None, C, W + 4, need, None) == dg.GEMM_ERR_MISALIGNED
        # a plan made without a device cannot run
        assert L.gemm_run(p, A, B, None, C, W, need, None) == dg.GEMM_ERR_NO_DEVICE
    finally:
        dg.gemm_plan_destroy(p)
    q = dg.int4_quant()
    p = dg.gemm_plan(16, 128, 256, ROW, COL, F16, U4, F16, 1, q)
    try:
        assert dg.lib().gemm_run(p, 0x10000, 0x20000, None, 0x30000, None, 0, None) == dg.GEMM_ERR_INVALID_ARG
    finally:
        dg.gemm_plan_destroy(p)


def test_query_and_destroy_null():
    assert dg.lib().gemm_plan_query(None, None) == dg.GEMM_ERR_INVALID_ARG
    assert dg.lib().gemm_workspace_size(None, None) == dg.GEMM_ERR_INVALID_ARG
    dg.gemm_plan_destroy(None)


@pytest.mark.parametrize("la,lb,bits", [(ROW, ROW, 1), (ROW, COL, 3), (COL, COL, 2)])
def test_direct_to_lds_plans(fake_cus, la, lb, bits):
    with env(DGEMM_FORCE_DTL=1, DGEMM_FORCE_MFMA=16):
        p = dg.gemm_plan(4096, 4096, 4096, la, lb, F16, F16, F16, 0)
        i = dg.gemm_plan_query(p)
        dg.gemm_plan_destroy(p)
    assert (i["direct_lds"], i["mfma_m"]) == (bits, 16)
    assert i["lds_pad_bytes"] == (0 if bits == 3 else 32)   # 16x16x32 kernels' transposed rows
    assert i["lds_bytes"] <= 160 * 1024
    with env(DGEMM_FORCE_DTL=1):   # both operands transposed: nothing to load directly
        with pytest.raises(dg.GemmError):
            dg.gemm_plan(4096, 4096, 4096, COL, ROW, F16, F16, F16, 0)


def test_pack_u4_tiled_places_every_group_of_every_column():
    # codes of column n, K group g (64 bytes of the column-major packing) go to the 4 KiB
    # block (n/64, g) at row n%64; every source byte lands exactly once
    N, K = 192, 384
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 256, size=N * K // 2, dtype=np.uint8)
    tiled = dg.gemm_pack_u4_tiled(codes, N, K)
    G = K // 128
    src = codes.reshape(N, G, 64)
    blocks = tiled.reshape(N // 64, G, 64, 64)
    for n in range(N):
        for g in range(G):
            assert np.array_equal(blocks[n // 64, g, n % 64], src[n, g]), (n, g)
    # a bijection on bytes: tagging every byte with its own index shows each moved once
    idx = np.arange(N * K // 2)
    moved = dg.gemm_pack_u4_tiled((idx % 251).astype(np.uint8), N, K)
    assert np.array_equal(np.sort(moved), np.sort((idx % 251).astype(np.uint8)))


def test_pack_u4_tiled_errors():
    L = dg.lib()
    buf = np.zeros(64 * 64, dtype=np.uint8)
    assert L.gemm_pack_u4_tiled(None, buf.ctypes.data, 64, 128) == dg.GEMM_ERR_INVALID_ARG
    assert L.gemm_pack_u4_tiled(buf.ctypes.data, buf.ctypes.data, 0, 128) == dg.GEMM_ERR_INVALID_ARG
    assert L.gemm_pack_u4_tiled(buf.ctypes.data, buf.ctypes.data, 32, 128) == dg.GEMM_ERR_UNSUPPORTED
    assert L.gemm_pack_u4_tiled(buf.ctypes.data, buf.ctypes.data, 64, 64) == dg.GEMM_ERR_UNSUPPORTED


def test_tiled_int4_plans(fake_cus):
    q = dg.int4_quant()
    T = dg.GEMM_U4_TILED
    assert _plan_status(16, 8192, 8192, ROW, T, F16, U4, F16, 0, quant=q)[0] == dg.GEMM_OK
    assert _plan_status(16, 8008, 8192, ROW, T, F16, U4, F16, 0, quant=q)[0] == dg.GEMM_ERR_UNSUPPORTED
    assert _plan_status(64, 64, 64, ROW, T, F16, F16, F16, 0)[0] == dg.GEMM_ERR_UNSUPPORTED
    assert _plan_status(64, 64, 64, ROW, 3, F16, F16, F16, 0)[0] == dg.GEMM_ERR_INVALID_ARG
    for M in (16, 4096):
        p = dg.gemm_plan(M, 8192, 8192, ROW, T, F16, U4, F16, 0, q)
        i = dg.gemm_plan_query(p)
        dg.gemm_plan_destroy(p)
        assert i["layout_b"] == T and i["kernel"] == (1 if M == 16 else 0)


F8 = dg.GEMM_F8


def test_fp8_plans(fake_cus):
    # every layout pair plans onto a 256x256 tile with a 128-K step; the transposed operand
    # gets the fp8 row permutation (256 rows, stride 16) and K-contiguous ones go straight
    # to LDS
    want_dtl = {(ROW, COL): 3, (COL, COL): 2, (ROW, ROW): 1, (COL, ROW): 0}
    for (la, lb), bits in want_dtl.items():
        p = dg.gemm_plan(4096, 4096, 4096, la, lb, F8, F8, F16, 0)
        i = dg.gemm_plan_query(p)
        dg.gemm_plan_destroy(p)
        assert (i["tile_m"], i["tile_n"], i["tile_k"], i["waves"], i["split_k"]) == (256, 256, 128, 8, 1)
        assert i["direct_lds"] == bits
        assert (i["perm_block"], i["perm_stride"]) == ((1, 1) if bits == 3 else (256, 16))
        assert i["lds_bytes"] <= 160 * 1024
    # contiguous extents in multiples of 16 bytes: 16 fp8 elements (8 are enough for fp16)
    assert _plan_status(64, 64, 24, ROW, COL, F8, F8, F16, 0)[0] == dg.GEMM_ERR_UNSUPPORTED
    assert _plan_status(64, 64, 24, ROW, COL, F16, F16, F16, 0)[0] == dg.GEMM_OK
    assert _plan_status(40, 64, 64, COL, COL, F8, F8, F16, 0)[0] == dg.GEMM_ERR_UNSUPPORTED
    assert _plan_status(64, 40, 64, ROW, ROW, F8, F8, F16, 0)[0] == dg.GEMM_ERR_UNSUPPORTED
    # K of two transposed operands is free; M <= 16 uses the tiled kernel
    assert _plan_status(48, 48, 37, COL, ROW, F8, F8, F32, 0)[0] == dg.GEMM_OK
    p = dg.gemm_plan(16, 8192, 4096, ROW, COL, F8, F8, F16, 0)
    i = dg.gemm_plan_query(p)
    dg.gemm_plan_destroy(p)
    assert i["kernel"] == 0 and i["tile_k"] == 128
    # fp8 output, mixed operand types and fp8 with int4 are not offered
    assert _plan_status(64, 64, 64, ROW, COL, F8, F8, F8, 0)[0] == dg.GEMM_ERR_UNSUPPORTED
    assert _plan_status(64, 64, 64, ROW, COL, F8, F16, F16, 0)[0] == dg.GEMM_ERR_UNSUPPORTED
    assert _plan_status(64, 64, 64, ROW, COL, F16, F8, F16, 0)[0] == dg.GEMM_ERR_UNSUPPORTED
    assert _plan_status(64, 64, 256, ROW, COL, F8, U4, F16, 0, quant=dg.int4_quant())[0] == dg.GEMM_ERR_UNSUPPORTED
    # split-K granule is the 128-K step
    p = dg.gemm_plan(16, 8192, 28672, ROW, COL, F8, F8, F16, 0)
    i = dg.gemm_plan_query(p)
    dg.gemm_plan_destroy(p)
    assert i["split_k"] == oracle.splitk_factor(16, 8192, 28672, 256, 256, 128, 256)


ATTN_HEADER = os.path.join(ROOT, "include", "dattn.h")


def test_attention_header_entry_point_is_exported():
    text = re.sub(r"/\*.*?\*/", "", open(ATTN_HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))
    assert names == ["attn_fwd"]
    lib = ctypes.CDLL(dg.LIB_PATH)
    for name in names:
        assert hasattr(lib, name), name


def test_attention_rejects_bad_arguments_before_any_device_work():
    L = dg.lib()
    P = 0x10000   # never dereferenced
    ok = (P, P + 0x100000, P + 0x200000, P + 0x300000, 2, 256, 256, 128, F16, 0.125, None)
    cases = [
        ((None,) + ok[1:], dg.GEMM_ERR_INVALID_ARG),
        (ok[:3] + (None,) + ok[4:], dg.GEMM_ERR_INVALID_ARG),
        (ok[:4] + (0,) + ok[5:], dg.GEMM_ERR_INVALID_ARG),
        (ok[:5] + (-1,) + ok[6:], dg.GEMM_ERR_INVALID_ARG),
        (ok[:6] + (0,) + ok[7:], dg.GEMM_ERR_INVALID_ARG),
        (ok[:8] + (9,) + ok[9:], dg.GEMM_ERR_INVALID_ARG),
        (ok[:9] + (float("nan"),) + ok[10:], dg.GEMM_ERR_INVALID_ARG),
        (ok[:9] + (float("inf"),) + ok[10:], dg.GEMM_ERR_INVALID_ARG),
        (ok[:7] + (64,) + ok[8:], dg.GEMM_ERR_UNSUPPORTED),            # head dim
        (ok[:8] + (dg.GEMM_F32,) + ok[9:], dg.GEMM_ERR_UNSUPPORTED),   # fp32 operands
        (ok[:8] + (F8,) + ok[9:], dg.GEMM_ERR_UNSUPPORTED),
        (ok[:4] + (64, 1 << 20) + ok[6:], dg.GEMM_ERR_UNSUPPORTED),    # Q beyond 2 GiB
        (ok[:4] + (64, 256, 1 << 20) + ok[7:], dg.GEMM_ERR_UNSUPPORTED),
        (ok[:4] + (1 << 31, 1 << 31) + ok[6:], dg.GEMM_ERR_UNSUPPORTED),   # products wrap
        (ok[:4] + (1, 1 << 62, 256) + ok[7:], dg.GEMM_ERR_UNSUPPORTED),
        (ok[:4] + (1 << 62, 1, 1) + ok[7:], dg.GEMM_ERR_UNSUPPORTED),
        (ok[:4] + (1, 1 << 23) + ok[6:], dg.GEMM_ERR_UNSUPPORTED),         # Q at 2 GiB
        ((P + 8,) + ok[1:], dg.GEMM_ERR_MISALIGNED),
        (ok[:3] + (P + 0x300002,) + ok[4:], dg.GEMM_ERR_MISALIGNED),
    ]
    for args, want in cases:
        assert L.attn_fwd(*args) == want, args
    import torch
    if not torch.cuda.is_available():
        assert L.attn_fwd(*ok) == dg.GEMM_ERR_NO_DEVICE
        # one row below the limit passes the size checks (and stops at the device)
        assert L.attn_fwd(*(ok[:4] + (1, (1 << 23) - 1, (1 << 23) - 1) + ok[7:])) == dg.GEMM_ERR_NO_DEVICE


class _FakeDeviceTensor:
    """Stands in for a device tensor of `nbytes` bytes (never dereferenced: the binding
    refuses it before calling the library)."""

    is_cuda = True

    def __init__(self, nbytes, contiguous=True):
        self.nbytes, self.contig = nbytes, contiguous

    def is_contiguous(self):
        return self.contig

    def numel(self):
        return self.nbytes // 2

    def element_size(self):
        return 2

    def data_ptr(self):
        return 0x10000


def test_binding_refuses_host_short_and_strided_tensors(fake_cus):
    import torch
    M = N = K = 64
    p = dg.gemm_plan(M, N, K, ROW, COL, F16, F16, F16, 1)
    try:
        full = M * K * 2
        dev = lambda n=full: _FakeDeviceTensor(n)
        cases = [
            ((torch.zeros(M * K, dtype=torch.int16), dev(), None, dev()), "device tensor"),
            ((dev(), dev(), None, dev(full - 2)), "bytes"),                      # C one short
            ((dev(full - 16), dev(), None, dev()), "bytes"),                     # A short
            ((dev(), _FakeDeviceTensor(full, contiguous=False), None, dev()), "contiguous"),
        ]
        for (A, B, S, C), msg in cases:
            with pytest.raises(ValueError, match=msg):
                dg.gemm_run(p, A, B, S, C, stream=0)
    finally:
        dg.gemm_plan_destroy(p)
    # int4 plans also size the scales: [K/group][N] fp16
    q = dg.int4_quant(64)
    p = dg.gemm_plan(16, 64, 256, ROW, COL, F16, "u4", F16, 1, q)
    try:
        with pytest.raises(ValueError, match="scales"):
            dg.gemm_run(p, _FakeDeviceTensor(16 * 256 * 2), _FakeDeviceTensor(64 * 128),
                        _FakeDeviceTensor((256 // 64) * 64 * 2 - 2), _FakeDeviceTensor(16 * 64 * 2),
                        stream=0)
    finally:
        dg.gemm_plan_destroy(p)
    # attention: every tensor at least BH x rows x D x 2 bytes
    ok = lambda rows: _FakeDeviceTensor(2 * rows * 128 * 2)
    with pytest.raises(ValueError, match="V"):
        dg.attn_fwd(ok(300), ok(500), _FakeDeviceTensor(2 * 500 * 128 * 2 - 2), ok(300),
                    2, 300, 500, 128, "f16", 0.125, stream=0)
    with pytest.raises(ValueError, match="device tensor"):
        dg.attn_fwd(ok(300), ok(500), ok(500), torch.zeros(2 * 300 * 128, dtype=torch.int16),
                    2, 300, 500, 128, "f16", 0.125, stream=0)


def test_pack_u4_tiled_refuses_a_short_array():
    codes = np.zeros(64 * 128 // 2 - 1, dtype=np.uint8)
    with pytest.raises(ValueError, match="N\\*K/2"):
        dg.gemm_pack_u4_tiled(codes, 64, 128)
