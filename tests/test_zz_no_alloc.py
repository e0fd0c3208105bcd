"""gemm_run_noalloc (the entry point that allocates nothing) against gemm_run, through the C ABI.

Each case plans a split-K GEMM, runs it once with gemm_run and a caller workspace, and then
twice in a row with gemm_run_noalloc, the second time on a smaller problem, so that the
second call sees the library's workspace as the first one left it. Random inputs; the
kernels and the summation order are the same, so the outputs must agree bit for bit.
"""
import numpy as np
import pytest

from dense_gemm_operand_amd import synth
from helpers import FMT_BYTES, to_dev

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)


def _inputs(seed, M, N, K, la, lb):
    rng = np.random.default_rng(seed)
    a = synth.to_bits(rng.standard_normal((M, K)) / 8, "f16")
    b = synth.to_bits(rng.standard_normal((K, N)) / 8, "f16")
    return synth.store(a, la), synth.store(b, lb)


def _run(noalloc, M, N, K, la, lb, sk, A, B, dtype_c="f32"):
    import torch
    import dense_gemm_operand_amd as dg
    plan = dg.gemm_plan(M, N, K, la, lb, "f16", "f16", dtype_c, sk)
    try:
        info = dg.gemm_plan_query(plan)
        dA, dB = to_dev(A), to_dev(B)
        eb = FMT_BYTES[dtype_c]
        C = torch.full((M * N,), 0x3A3A, dtype=torch.int32 if eb == 4 else torch.int16, device="cuda")
        if noalloc:
            dg.gemm_run_noalloc(plan, dA, dB, None, C)
        else:
            nws = dg.gemm_workspace_size(plan)
            ws = torch.zeros(max(nws, 16), dtype=torch.uint8, device="cuda")
            dg.gemm_run(plan, dA, dB, None, C, ws if nws else None)
        torch.cuda.synchronize()
        return C.cpu().numpy().copy(), info
    finally:
        dg.gemm_plan_destroy(plan)


CASES = [
    # (first problem, second smaller problem): (M, N, K, layout A, layout B, split_k)
    ((16, 2048, 8192, "row", "col", 4), (8, 1000, 4104, "row", "col", 2)),     # skinny kernel
    ((512, 512, 4096, "col", "col", 4), (296, 200, 1000, "col", "col", 2)),    # tiled kernel
    ((16, 4096, 16384, "row", "col", 16), (16, 4096, 16384, "row", "col", 1)),  # no workspace
]


@pytest.mark.parametrize("first,second", CASES)
def test_noalloc_matches_gemm_run_on_two_calls(first, second):
    outs = {}
    for i, (M, N, K, la, lb, sk) in enumerate((first, second)):
        _say("noalloc", i, M, N, K, la, lb, sk)
        A, B = _inputs(100 + i, M, N, K, la, lb)
        ref, info = _run(False, M, N, K, la, lb, sk, A, B)
        assert info["split_k"] == sk
        outs[i] = (ref, _run(True, M, N, K, la, lb, sk, A, B)[0])
    for i in (0, 1):
        ref, got = outs[i]
        assert np.array_equal(ref, got), f"call {i}: {int((ref != got).sum())} elements differ"


def test_noalloc_refuses_a_workspace_beyond_its_limit():
    import dense_gemm_operand_amd as dg
    # 16 splits of 256 tiles of 256 x 256 fp32 partials: far beyond 32 MiB
    plan = dg.gemm_plan(4096, 4096, 8192, "row", "col", "f16", "f16", "f16", 16)
    try:
        assert dg.gemm_workspace_size(plan) > dg.NOALLOC_WORKSPACE_BYTES
        st = dg.lib().gemm_run_noalloc(plan, 0x1000, 0x1000, None, 0x1000, None)
        assert st == dg.GEMM_ERR_WORKSPACE_TOO_SMALL
    finally:
        dg.gemm_plan_destroy(plan)
