"""GPU parity of the fp8 (OCP E4M3) operand path against the CPU oracle.

Small integers are exact E4M3 values and their products and sums stay exact in fp32, so
with integer inputs the GPU result must equal the oracle bit for bit for every layout,
ragged shape and split; random N(0, 1) inputs (rounded to E4M3) must meet the acceptance
bar. At the 4096^3 size the bench runs, sampled rows are checked against the oracle and a
permutation matrix as one operand must give an exact permutation of the other."""
import numpy as np
import pytest

import oracle
from dense_gemm_operand_amd import synth
from helpers import check_tolerance, operand_max, reference, run_gpu

pytestmark = pytest.mark.gpu

LAYOUTS = [("row", "row"), ("row", "col"), ("col", "row"), ("col", "col")]


def _say(*a):
    print("[case]", *a, flush=True)


def _inputs_int(M, N, K, la, lb, seed, lo=-8, hi=8):
    rng = np.random.default_rng(seed)
    a = synth.integer_matrix(rng, M, K, lo, hi, "f8")
    b = synth.integer_matrix(rng, K, N, lo, hi, "f8")
    return {"M": M, "N": N, "K": K, "layout_a": la, "layout_b": lb,
            "A": synth.store(a, la), "B": synth.store(b, lb)}


def _inputs_rand(M, N, K, la, lb, seed, dist="normal1"):
    w = synth.Workload("t", 0, M, N, K, la, lb, "f8", "f16", dist)
    return synth.make_inputs(w, seed=seed)


@pytest.mark.parametrize("sched", [1, 0])
@pytest.mark.parametrize("M,N,K", [(400, 656, 208), (272, 528, 1040)])
@pytest.mark.parametrize("la,lb", LAYOUTS)
def test_fp8_integer_inputs_bit_exact(M, N, K, la, lb, sched):
    # several 256x256 tiles with ragged edges in M and N; K ragged inside a 128 step, and an
    # odd number of steps (the loop's padding step must add nothing); the ping-pong (1,
    # default) and the software-pipeline (0) schedule
    from helpers import env
    _say("f8 int", la, lb, M, N, K, sched)
    inp = _inputs_int(M, N, K, la, lb, seed=201)
    with env(DGEMM_FORCE_SCHED=sched):
        c, info = run_gpu(inp, "f8", "f32", split_k=1, guard=64)
    assert (info["tile_m"], info["tile_n"], info["tile_k"]) == (256, 256, 128)
    _, ref = reference(inp, "f8", "f32")
    assert np.array_equal(c, ref)


@pytest.mark.parametrize("la,lb", LAYOUTS)
@pytest.mark.parametrize("out", ["f16", "f32", "bf16"])
def test_fp8_random_inputs_within_tolerance(la, lb, out):
    M, N, K = 528, 400, 336
    _say("f8 rand", la, lb, out)
    inp = _inputs_rand(M, N, K, la, lb, seed=211)
    c, _ = run_gpu(inp, "f8", out, split_k=1, guard=32)
    _, ref = reference(inp, "f8", out)
    amax, bmax = operand_max(inp, "f8")
    check_tolerance(c, ref, out, K, amax, bmax, f"f8 {la}/{lb} -> {out}")


@pytest.mark.parametrize("sk", [2, 4, 8, 16])
@pytest.mark.parametrize("la,lb", [("col", "col"), ("col", "row")])
def test_fp8_split_k_integer_identical(sk, la, lb):
    M, N, K = 288, 272, 2064
    _say("f8 split", sk, la, lb)
    inp = _inputs_int(M, N, K, la, lb, seed=221)
    c, info = run_gpu(inp, "f8", "f32", split_k=sk, guard=16)
    assert info["split_k"] == sk
    _, ref = reference(inp, "f8", "f32")
    assert np.array_equal(c, ref)


@pytest.mark.parametrize("M,N,K", [(16, 16, 16), (48, 48, 37), (272, 16, 144), (16, 272, 1)])
@pytest.mark.parametrize("la,lb", LAYOUTS)
def test_fp8_tiles_mostly_out_of_range(M, N, K, la, lb):
    # one tile almost entirely past M, N or K; K need not be a multiple of 16 only when
    # neither operand is K-contiguous
    kc = la == "row" or lb == "col"
    if kc and K % 16:
        pytest.skip("a K-contiguous fp8 operand needs K % 16 == 0")
    _say("f8 edge", M, N, K, la, lb)
    inp = _inputs_int(M, N, K, la, lb, seed=231)
    c, _ = run_gpu(inp, "f8", "f32", split_k=1, guard=32)
    _, ref = reference(inp, "f8", "f32")
    assert np.array_equal(c, ref)


def test_fp8_special_values():
    # the extreme finite magnitudes and subnormals decode and multiply correctly, and a NaN
    # code (0x7F) in a row of A makes exactly that row NaN
    M, N, K = 256, 256, 128
    rng = np.random.default_rng(241)
    vals = np.array([448.0, -448.0, 2.0 ** -9, -(2.0 ** -9), 2.0 ** -6, 240.0, 0.0, 1.0])
    a = rng.choice(vals, size=(M, K))
    b = rng.choice(vals, size=(K, N))
    abits, bbits = synth.to_bits(a, "f8"), synth.to_bits(b, "f8")
    assert np.array_equal(oracle.decode(abits, "f8"), a)
    abits[5, 7] = 0x7F
    inp = {"M": M, "N": N, "K": K, "layout_a": "col", "layout_b": "col",
           "A": synth.store(abits, "col"), "B": synth.store(bbits, "col")}
    c, _ = run_gpu(inp, "f8", "f32", split_k=1, guard=16)
    g = oracle.decode(c, "f32")
    nan_rows = np.where(np.isnan(g).any(axis=1))[0]
    assert list(nan_rows) == [5] and np.isnan(g[5]).all()
    _, ref = reference(inp, "f8", "f32")
    keep = np.arange(M) != 5
    # products span 2^-18 .. 2^17.6, so fp32 sums round; the other rows meet the bar
    check_tolerance(c[keep], ref[keep], "f32", K, 448.0, 448.0, "f8 special")


@pytest.mark.parametrize("la,lb", LAYOUTS)
def test_fp8_full_size_sampled_rows(la, lb):
    # 4096^3 as the bench runs it (N(0, 1) inputs rounded to E4M3, fp16 C)
    w = synth.WORKLOADS["square_4096_f8"]
    _say("f8 full", la, lb)
    inp = synth.make_inputs(w, layout_a=la, layout_b=lb)
    c, info = run_gpu(inp, "f8", w.dtype_c, split_k=w.split_k, guard=16)
    amax, bmax = operand_max(inp, "f8")
    M = inp["M"]
    for r0, r1 in [(0, 8), (2052, 2060), (M - 8, M)]:
        _, ref = reference(inp, "f8", w.dtype_c, rows=(r0, r1))
        check_tolerance(c[r0:r1], ref, w.dtype_c, inp["K"], amax, bmax, f"f8 full rows {r0}..{r1}")


@pytest.mark.parametrize("which", ["A", "B"])
@pytest.mark.parametrize("la,lb", LAYOUTS)
def test_fp8_full_size_permutation_every_element(which, la, lb):
    n = 4096
    _say("f8 full perm", which, la, lb)
    rng = np.random.default_rng(251 + (which == "B"))
    perm = rng.permutation(n)
    other = synth.integer_matrix(rng, n, n, -16, 16, "f8")
    pm = np.zeros((n, n))
    pm[np.arange(n), perm] = 1.0
    pbits = synth.to_bits(pm, "f8")
    a, b = (pbits, other) if which == "A" else (other, pbits)
    inp = {"M": n, "N": n, "K": n, "layout_a": la, "layout_b": lb,
           "A": synth.store(a, la), "B": synth.store(b, lb)}
    c, _ = run_gpu(inp, "f8", "f16", split_k=1, guard=16)
    # A = P: C[i, :] = B[perm[i], :]; B = P: C[:, perm[k]] = A[:, k]
    o = oracle.decode(other, "f8")
    if which == "A":
        want = o[perm]
    else:
        inv = np.empty(n, dtype=np.int64)
        inv[perm] = np.arange(n)
        want = o[:, inv]
    assert np.array_equal(oracle.decode(c, "f16"), want)
