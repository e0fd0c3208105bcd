"""GPU parity at the workloads' full sizes, in the launch configuration the bench times.

Every workload is planned as bench.py plans it (same seeded inputs, same split-K request,
so the same kernel, tile and split). Random inputs are checked against the oracle to the
acceptance bar on every output row, except for the int4 M=4096 product (550 GFLOP, minutes
of oracle time), which is checked on sampled row ranges (first rows, a middle range, last
rows: several tiles and the edge). Properties that hold at any size are checked on every element of
the full-size result: a permutation matrix as A (or B) makes C an exact row (or column)
permutation of the other operand, and unit rows of A make C the exactly dequantised int4
weight rows."""
import numpy as np
import pytest

import oracle
from dense_gemm_operand_amd import synth
from helpers import check_tolerance, env, operand_max, reference, run_gpu

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)


def _row_ranges(M: int, n: int = 8):
    if M <= 3 * n:
        return [(0, M)]
    mid = (M // 2) // n * n + n // 2   # off the tile grid
    return [(0, n), (mid, mid + n), (M - n, M)]


def _check_sampled(inp, w, c, what):
    amax, bmax = operand_max(inp, w.dtype_ab, int4=w.int4)
    for r0, r1 in _row_ranges(inp["M"]):
        _, ref = reference(inp, w.dtype_ab, w.dtype_c, int4=w.int4, rows=(r0, r1))
        check_tolerance(c[r0:r1], ref, w.dtype_c, inp["K"], amax, bmax, f"{what} rows {r0}..{r1}")


FULL = [("square_tt_256", None, None), ("square_4096", "col", "col"),
        ("square_4096", "col", "row"), ("square_4096", "row", "col"),
        ("square_4096", "row", "row"), ("nonpow2_bf16", None, None),
        ("skinny_splitk", None, None), ("int4_m16", None, None)]


@pytest.mark.parametrize("name,la,lb", FULL)
def test_full_size_every_row_against_the_oracle(name, la, lb):
    w = synth.WORKLOADS[name]
    _say("full", name, la, lb)
    inp = synth.make_inputs(w, layout_a=la, layout_b=lb)
    c, info = run_gpu(inp, w.dtype_ab, w.dtype_c, split_k=w.split_k, int4=w.int4, guard=16)
    amax, bmax = operand_max(inp, w.dtype_ab, int4=w.int4)
    _, ref = reference(inp, w.dtype_ab, w.dtype_c, int4=w.int4)
    rel, worst = check_tolerance(c, ref, w.dtype_c, inp["K"], amax, bmax, name)
    _say(f"  relative Frobenius error {rel:.3e}, largest element error {worst:.3e} "
         f"(bound {4e-3 * np.sqrt(inp['K']) * amax * bmax:.3e})")


def test_full_size_nonpow2_tile_every_row():
    # the 3072 x 5120 x 6144 bf16 shape on the non-power-of-2 192 x 320 tile (16 x 16 = 256
    # tiles for 256 CUs; the default plan takes 256 x 256), every row against the oracle
    w = synth.WORKLOADS["nonpow2_bf16"]
    _say("full nonpow2 192x320")
    inp = synth.make_inputs(w)
    c, info = run_gpu(inp, w.dtype_ab, w.dtype_c, split_k=1, force_tile="192x320", guard=16)
    assert (info["tile_m"], info["tile_n"], info["grid_x"]) == (192, 320, 256)
    amax, bmax = operand_max(inp, w.dtype_ab)
    _, ref = reference(inp, w.dtype_ab, w.dtype_c)
    check_tolerance(c, ref, w.dtype_c, inp["K"], amax, bmax, "192x320")


def test_full_size_sampled_rows_int4_m4096():
    w = synth.WORKLOADS["int4_m4096"]
    _say("full sampled", w.name)
    inp = synth.make_inputs(w)
    c, info = run_gpu(inp, w.dtype_ab, w.dtype_c, split_k=w.split_k, int4=w.int4, guard=16)
    _check_sampled(inp, w, c, w.name)


def test_full_size_split_k_sweep():
    # the split-K shape with every factor the pages' heuristic can pick, plus the auto choice
    w = synth.WORKLOADS["skinny_splitk"]
    inp = synth.make_inputs(w)
    _, ref = reference(inp, w.dtype_ab, w.dtype_c)
    amax, bmax = operand_max(inp, w.dtype_ab)
    for sk in (0, 1, 2, 4, 8, 16):
        _say("full split-k", sk)
        c, info = run_gpu(inp, w.dtype_ab, w.dtype_c, split_k=sk, guard=16)
        assert sk == 0 or info["split_k"] == sk
        check_tolerance(c, ref, w.dtype_c, inp["K"], amax, bmax, f"split_k={sk}")


def _perm_inputs(which: str, la: str, lb: str, seed: int):
    n = 4096
    rng = np.random.default_rng(seed)
    perm = rng.permutation(n)
    other = synth.integer_matrix(rng, n, n, -8, 8, "f16")
    pm = np.zeros((n, n))
    pm[np.arange(n), perm] = 1.0
    pbits = synth.to_bits(pm, "f16")
    a, b = (pbits, other) if which == "A" else (other, pbits)
    inp = {"M": n, "N": n, "K": n, "layout_a": la, "layout_b": lb,
           "A": synth.store(a, la), "B": synth.store(b, lb)}
    # A = P: C[i, :] = B[perm[i], :]; B = P: C[:, perm[k]] = A[:, k], i.e. C = A[:, inv]
    if which == "A":
        want = other[perm]
    else:
        inv = np.empty(n, dtype=np.int64)
        inv[perm] = np.arange(n)
        want = other[:, inv]
    return inp, want


@pytest.mark.parametrize("which", ["A", "B"])
@pytest.mark.parametrize("la,lb", [("col", "col"), ("col", "row"), ("row", "col"), ("row", "row")])
@pytest.mark.parametrize("loader", ["default", "transposing_reads", "in_register", "in_register_16x16"])
def test_full_size_permutation_every_element(which, la, lb, loader):
    # 4096^3 as the bench runs it: every element of C must be the exact permuted entry
    if loader == "transposing_reads" and la == "row" and lb == "col":
        pytest.skip("no transposed operand")
    if loader == "in_register" and (la, lb) != ("col", "row"):
        pytest.skip("NN's default transposes in registers; TT's is the next case")
    if loader == "in_register_16x16" and (la, lb) != ("row", "row"):
        pytest.skip("TT's in-register transpose on 16x16x32 blocks (NN's is its default)")
    _say("full perm", which, la, lb, loader)
    inp, want = _perm_inputs(which, la, lb, seed=111 + (which == "B"))
    force = {"default": {}, "transposing_reads": {"DGEMM_FORCE_DTL": 2},
             "in_register": {"DGEMM_FORCE_DTL": 0},
             "in_register_16x16": {"DGEMM_FORCE_DTL": 1, "DGEMM_FORCE_MFMA": 16}}[loader]
    with env(**force):
        c, info = run_gpu(inp, "f16", "f16", split_k=1, guard=16)
    # NT and TT (a transposed B) take the transposing reads by default
    want_tr = loader == "transposing_reads" or (loader == "default" and lb == "row")
    assert ((info["direct_lds"] & 12) != 0) == want_tr
    if loader == "in_register_16x16":
        assert info["mfma_m"] == 16
    assert np.array_equal(c, want)


@pytest.mark.parametrize("name", ["int4_m16", "int4_m4096"])
def test_full_size_int4_unit_rows_give_dequantised_weights(name):
    # the int4 shapes' own codes and scales; A rows are unit vectors, so each C row is one
    # dequantised weight row, exactly (one nonzero product per sum)
    w = synth.WORKLOADS[name]
    _say("full int4 unit rows", name)
    inp = synth.make_inputs(w)
    M, K, N = inp["M"], inp["K"], inp["N"]
    rng = np.random.default_rng(121)
    pick = rng.integers(0, K, size=M)
    a = np.zeros((M, K))
    a[np.arange(M), pick] = 1.0
    inp["A"] = synth.store(synth.to_bits(a, "f16"), "row")
    c, info = run_gpu(inp, "f16", "f16", split_k=w.split_k, int4=True, guard=16)
    wts = oracle.dequant_u4(inp["B"], inp["scales"], K, N)
    assert np.array_equal(oracle.decode(c, "f16"), wts[pick])


@pytest.mark.parametrize("name", ["int4_m16", "int4_m4096"])
def test_full_size_int4_tiled_layout(name):
    # the int4 shapes with their codes pre-tiled: sampled rows against the oracle (which reads
    # the column-major packing) and unit rows giving the exact dequantised weights
    import dense_gemm_operand_amd as dg
    w = synth.WORKLOADS[name]
    _say("full int4 tiled", name)
    inp = synth.make_inputs(w)
    M, K, N = inp["M"], inp["K"], inp["N"]
    tiled = dict(inp, B=dg.gemm_pack_u4_tiled(inp["B"], N, K), layout_b="u4_tiled")
    c, info = run_gpu(tiled, "f16", "f16", split_k=w.split_k, int4=True, guard=16)
    assert info["layout_b"] == dg.GEMM_U4_TILED
    _check_sampled(inp, w, c, name + " tiled")
    rng = np.random.default_rng(141)
    pick = rng.integers(0, K, size=M)
    a = np.zeros((M, K))
    a[np.arange(M), pick] = 1.0
    tiled["A"] = synth.store(synth.to_bits(a, "f16"), "row")
    c, _ = run_gpu(tiled, "f16", "f16", split_k=w.split_k, int4=True, guard=16)
    wts = oracle.dequant_u4(inp["B"], inp["scales"], K, N)
    assert np.array_equal(oracle.decode(c, "f16"), wts[pick])
