"""LDS-race check: the tiled kernels against an over-synchronised build of themselves.

libdgemm_oversync.so is built from the same sources with DGEMM_OVERSYNC=1: in the main loops
every phase ends with a wait for every outstanding load and LDS access and a workgroup
barrier. It adds the same products in the same order, so on the same inputs its output
must equal the normal build's bit for bit. The normal build orders its direct-to-LDS loads,
LDS stores and fragment reads by hand (partial waits, one barrier per phase or step); a
missing wait or barrier there would let a wave read a tile that is not yet (or no longer)
in LDS, and the two builds would then differ. Random inputs (so that a stale or early tile
changes the result), ragged shapes that span several tiles, both main-loop schedules, all
three operand loaders, every layout pair they serve, split-K with partial chunks, fp16 and
bf16, and fp8.
"""
import contextlib

import numpy as np
import pytest

from dense_gemm_operand_amd import build as dg_build
from dense_gemm_operand_amd import synth
from helpers import env, run_gpu

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)


@contextlib.contextmanager
def library(path):
    """Route the binding to another build of the library for the duration."""
    import dense_gemm_operand_amd as dg
    saved = dg.LIB_PATH, dg._lib
    dg.LIB_PATH, dg._lib = path, None
    try:
        yield
    finally:
        dg.LIB_PATH, dg._lib = saved


def _inputs(M, N, K, la, lb, fmt, seed):
    rng = np.random.default_rng(seed)
    a = synth.to_bits(rng.standard_normal((M, K)) / 4, fmt)
    b = synth.to_bits(rng.standard_normal((K, N)) / 4, fmt)
    return {"M": M, "N": N, "K": K, "layout_a": la, "layout_b": lb,
            "A": synth.store(a, la), "B": synth.store(b, lb)}


def _both(inp, fmt, out, hooks, split_k=1, tile="256x256"):
    with env(**hooks):
        ref, info = run_gpu(inp, fmt, out, split_k=split_k, guard=8, force_tile=tile)
        with library(dg_build.LIB_OVERSYNC):
            got, info2 = run_gpu(inp, fmt, out, split_k=split_k, guard=8, force_tile=tile)
    keys = ("tile_m", "tile_n", "waves", "schedule", "direct_lds", "split_k")
    assert {k: info[k] for k in keys} == {k: info2[k] for k in keys}
    assert f"{info['tile_m']}x{info['tile_n']}" == tile
    return ref, got, info


LAYOUTS = [("col", "col"), ("col", "row"), ("row", "col"), ("row", "row")]
# (schedule, loader): loader 0 = transposed operands through registers, 1 = K-contiguous
# operands straight into LDS, 2 = transposed operands straight into LDS, transposed by the reads
SCHED_LOADER = [(1, 1), (1, 2), (1, 0), (0, 0), (0, 1), (0, 2), (2, 1), (2, 2)]
# the 16x16x32 ping-pong at 256x256 (loader 1: K-contiguous operands direct, transposed
# ones through the in-register transpose; loader 2: every operand direct)
SCHED_LOADER16 = [(1, 1), (1, 2)]


def _served(sched, loader, la, lb, tile="256x256"):
    transposed = la == "col" or lb == "row"
    kcontig = la == "row" or lb == "col"
    if sched == 2 or tile == "192x320" and sched == 1:
        # every operand direct: loader 1 for TN, loader 2 wherever one is transposed
        return transposed if loader == 2 else (loader == 1 and not transposed)
    return {0: True, 1: kcontig, 2: transposed}[loader]


@pytest.mark.parametrize("sched,loader,mfma", [(s, l, 32) for s, l in SCHED_LOADER] +
                         [(s, l, 16) for s, l in SCHED_LOADER16])
@pytest.mark.parametrize("la,lb", LAYOUTS)
def test_oversynchronised_build_bit_identical(sched, loader, mfma, la, lb):
    # (with loader 2 the 16x16x32 ping-pong loads every operand directly, as schedule 2 does)
    if not _served(2 if (mfma == 16 and loader == 2) else sched, loader, la, lb):
        pytest.skip("this loader serves no operand of this layout pair")
    M, N, K = 520, 264, 712   # 3 x 2 tiles of 256 x 256, ragged edges, 11 K steps + a tail
    _say("oversync", sched, loader, mfma, la, lb)
    inp = _inputs(M, N, K, la, lb, "f16", seed=301 + 7 * sched + loader)
    ref, got, info = _both(inp, "f16", "f32", {"DGEMM_FORCE_SCHED": sched, "DGEMM_FORCE_DTL": loader,
                                               "DGEMM_FORCE_MFMA": mfma})
    assert info["schedule"] == sched and info["mfma_m"] == mfma
    assert np.array_equal(ref, got), f"{int((ref != got).sum())} of {ref.size} elements differ"


@pytest.mark.parametrize("sched,loader", [(1, 2), (1, 1), (0, 2), (2, 2), (2, 1)])
@pytest.mark.parametrize("la,lb", LAYOUTS)
def test_oversynchronised_build_bit_identical_nonpow2_tile(sched, loader, la, lb):
    # the 192 x 320 tile with direct-to-LDS loads (64-wide K-row segments for transposed
    # operands): 2 x 3 tiles with ragged edges, 10 K steps and a tail
    if not _served(sched, loader, la, lb, "192x320"):
        pytest.skip("this loader serves no operand of this layout pair")
    M, N, K = 392, 720, 680
    _say("oversync 192x320", sched, loader, la, lb)
    inp = _inputs(M, N, K, la, lb, "bf16", seed=341 + 7 * sched + loader)
    ref, got, info = _both(inp, "bf16", "f32", {"DGEMM_FORCE_SCHED": sched, "DGEMM_FORCE_DTL": loader},
                           tile="192x320")
    assert (info["tile_m"], info["schedule"]) == (192, sched)
    assert np.array_equal(ref, got), f"{int((ref != got).sum())} of {ref.size} elements differ"


@pytest.mark.parametrize("la,lb,fmt", [("col", "row", "bf16"), ("row", "col", "bf16"), ("col", "col", "f8"),
                                       ("row", "row", "f8")])
@pytest.mark.parametrize("split_k", [1, 2])
def test_oversynchronised_build_bit_identical_defaults(la, lb, fmt, split_k):
    # the default plan of each type, also with split-K (two splits of a K that is not a
    # multiple of the step: the second chunk is partial)
    M, N, K = 304, 528, 1008
    _say("oversync default", la, lb, fmt, split_k)
    inp = _inputs(M, N, K, la, lb, fmt, seed=331 + split_k)
    ref, got, _ = _both(inp, fmt, "f32", {}, split_k=split_k)
    assert np.array_equal(ref, got), f"{int((ref != got).sum())} of {ref.size} elements differ"
