"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Integer-valued inputs make every partial sum exact in fp32, so the GPU result must equal
the oracle bit for bit whatever the layout, tile, permutation or split; random inputs
must meet the acceptance bar (relative Frobenius <= 1e-3 against the oracle rounded to
the output format, every element within 4e-3 * sqrt(K) * max|a| * max|b|)."""
import numpy as np
import pytest

import oracle
from dense_gemm_operand_amd import synth
from helpers import check_tolerance, operand_max, reference, run_gpu

pytestmark = pytest.mark.gpu

LAYOUTS = [("row", "row"), ("row", "col"), ("col", "row"), ("col", "col")]
TILES = ["256x256", "192x320", "128x128", "64x64"]


def _inputs_int(M, N, K, la, lb, fmt, seed, lo=-2, hi=2):
    rng = np.random.default_rng(seed)
    a = synth.integer_matrix(rng, M, K, lo, hi, fmt)
    b = synth.integer_matrix(rng, K, N, lo, hi, fmt)
    return {"M": M, "N": N, "K": K, "layout_a": la, "layout_b": lb,
            "A": synth.store(a, la), "B": synth.store(b, lb)}


def _inputs_rand(M, N, K, la, lb, fmt, seed, dist="normal_sqrtk"):
    w = synth.Workload("t", 0, M, N, K, la, lb, fmt, fmt, dist)
    return synth.make_inputs(w, seed=seed)


def _say(*a):
    print("[case]", *a, flush=True)


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("la,lb", LAYOUTS)
@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_integer_inputs_bit_exact_every_layout_and_tile(tile, la, lb, fmt):
    # several tiles in each direction plus ragged tails in M, N and K
    M, N, K = 392 + 8, 648, 200
    _say("int", tile, la, lb, fmt, M, N, K)
    inp = _inputs_int(M, N, K, la, lb, fmt, seed=21)
    c, info = run_gpu(inp, fmt, "f32", split_k=1, force_tile=tile, guard=64)
    assert f"{info['tile_m']}x{info['tile_n']}" == tile
    _, ref = reference(inp, fmt, "f32")
    assert np.array_equal(c, ref)


@pytest.mark.parametrize("la,lb", LAYOUTS)
@pytest.mark.parametrize("fmt,out", [("f16", "f16"), ("f16", "f32"), ("bf16", "bf16"),
                                     ("bf16", "f32"), ("f16", "bf16")])
def test_random_inputs_within_tolerance(la, lb, fmt, out):
    M, N, K = 520, 392, 328
    _say("rand", la, lb, fmt, out)
    inp = _inputs_rand(M, N, K, la, lb, fmt, seed=31)
    c, _ = run_gpu(inp, fmt, out, split_k=1, guard=32)
    _, ref = reference(inp, fmt, out)
    amax, bmax = operand_max(inp, fmt)
    check_tolerance(c, ref, out, K, amax, bmax, f"{la}/{lb} {fmt}->{out}")


@pytest.mark.parametrize("sk", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("la,lb", [("row", "row"), ("col", "col")])
def test_split_k_integer_identical_for_every_factor(sk, la, lb):
    M, N, K = 264, 136, 1096
    _say("splitk-tile", sk, la, lb)
    inp = _inputs_int(M, N, K, la, lb, "f16", seed=41, lo=-3, hi=3)
    c, info = run_gpu(inp, "f16", "f32", split_k=sk, force_tile="128x128", guard=16)
    assert info["split_k"] == sk
    _, ref = reference(inp, "f16", "f32")
    assert np.array_equal(c, ref)


def test_split_k_random_deterministic_and_within_tolerance():
    M, N, K = 304, 200, 4000
    _say("splitk-determinism")
    inp = _inputs_rand(M, N, K, "col", "row", "bf16", seed=42, dist="normal002")
    outs, info = run_gpu(inp, "bf16", "bf16", split_k=8, repeat=3, force_tile="128x128")
    assert info["split_k"] == 8
    assert all(np.array_equal(outs[0], o) for o in outs[1:])
    _, ref = reference(inp, "bf16", "bf16")
    amax, bmax = operand_max(inp, "bf16")
    check_tolerance(outs[0], ref, "bf16", K, amax, bmax, "split-K bf16")


def test_split_k_with_empty_splits():
    # K = 256 in 16 splits of 64: four splits hold all of K, twelve are empty
    M, N, K = 128, 128, 256
    _say("empty-splits")
    inp = _inputs_int(M, N, K, "row", "row", "f16", seed=43)
    c, info = run_gpu(inp, "f16", "f32", split_k=16, force_tile="128x128")
    _, ref = reference(inp, "f16", "f32")
    assert np.array_equal(c, ref)


@pytest.mark.parametrize("sched", [1, 0])
@pytest.mark.parametrize("la,lb", LAYOUTS)
def test_split_k_with_empty_splits_256_tiles(la, lb, sched):
    # the 256x256 kernels (ping-pong, the default, and the pipeline): K = 256 in 16 splits of
    # 64, so twelve splits run no K step at all (zero sums through the fix-up)
    from helpers import env
    M, N, K = 264, 136, 256
    _say("empty-splits-256", la, lb, sched)
    inp = _inputs_int(M, N, K, la, lb, "f16", seed=44)
    with env(DGEMM_FORCE_SCHED=sched):
        c, info = run_gpu(inp, "f16", "f32", split_k=16, force_tile="256x256", guard=16)
    assert info["split_k"] == 16 and info["tile_m"] == 256
    _, ref = reference(inp, "f16", "f32")
    assert np.array_equal(c, ref)


@pytest.mark.parametrize("M,N,K", [(16, 8192 // 8, 28672 // 8), (1, 200, 4104), (4, 1, 4096),
                                   (1, 1, 4096), (13, 24, 264)])
@pytest.mark.parametrize("sk", [0, 1, 4])
def test_skinny_integer_bit_exact(M, N, K, sk):
    _say("skinny-int", M, N, K, sk)
    inp = _inputs_int(M, N, K, "row", "col", "f16", seed=51, lo=-4, hi=4)
    c, info = run_gpu(inp, "f16", "f32", split_k=sk, guard=8)
    assert info["kernel"] == 1
    _, ref = reference(inp, "f16", "f32")
    assert np.array_equal(c, ref)


def test_reduction_shapes_of_the_cross_wave_reduce():
    # 4096 -> 1 and 4 x 4096 -> 4 sums (IREE PR 19596 test cases) as products with ones
    for M in (1, 4):
        _say("reduce", M)
        rng = np.random.default_rng(52 + M)
        a = synth.integer_matrix(rng, M, 4096, -8, 8, "f16")
        ones = synth.to_bits(np.ones((4096, 1)), "f16")
        inp = {"M": M, "N": 1, "K": 4096, "layout_a": "row", "layout_b": "col",
               "A": synth.store(a, "row"), "B": synth.store(ones, "col")}
        c, info = run_gpu(inp, "f16", "f32", split_k=0)
        want = oracle.decode(a, "f16").sum(axis=1)
        assert np.array_equal(oracle.decode(c, "f32")[:, 0], want)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_skinny_random_within_tolerance(fmt):
    M, N, K = 16, 1024, 7168
    _say("skinny-rand", fmt)
    inp = _inputs_rand(M, N, K, "row", "col", fmt, seed=53, dist="uniform05")
    c, info = run_gpu(inp, fmt, fmt, split_k=0)
    _, ref = reference(inp, fmt, fmt)
    amax, bmax = operand_max(inp, fmt)
    check_tolerance(c, ref, fmt, K, amax, bmax, "skinny")


def _int4_inputs(M, N, K, seed, la="row"):
    w = synth.WORKLOADS["int4_m16"]
    inp = synth.make_inputs(w, M=M, N=N, K=K, seed=seed, layout_a=la)
    return inp


@pytest.mark.parametrize("M", [16, 256])
def test_int4_dequant_bit_exact_through_identity_rows(M):
    # A = unit rows picking K indices, so C rows are dequantised weight rows, exactly
    N, K = 320, 512
    _say("int4-identity", M)
    inp = _int4_inputs(M, N, K, seed=61)
    pick = np.random.default_rng(62).choice(K, size=M, replace=False)
    a = np.zeros((M, K))
    a[np.arange(M), pick] = 1.0
    inp["A"] = synth.store(synth.to_bits(a, "f16"), "row")
    c, info = run_gpu(inp, "f16", "f16", split_k=1, int4=True)
    w = oracle.dequant_u4(inp["B"], inp["scales"], K, N)
    assert np.array_equal(oracle.decode(c, "f16"), w[pick])


@pytest.mark.parametrize("M,la", [(16, "row"), (8, "row"), (384, "row"), (384, "col")])
def test_int4_random_within_tolerance(M, la):
    N, K = 512, 1024
    _say("int4-rand", M, la)
    inp = _int4_inputs(M, N, K, seed=63, la=la)
    c, info = run_gpu(inp, "f16", "f16", split_k=0, int4=True, guard=8)
    _, ref = reference(inp, "f16", "f16", int4=True)
    amax, bmax = operand_max(inp, "f16", int4=True)
    check_tolerance(c, ref, "f16", K, amax, bmax, "int4")


@pytest.mark.parametrize("dt,la,lb", [("f16", "col", "col"), ("bf16", "col", "row")])
@pytest.mark.parametrize("no_perm", [1, 2])
def test_no_permutation_variant_matches(dt, la, lb, no_perm):
    # the identity-row-order variants (padded rows, and unpadded 128-byte rows) give the
    # same bits as the permuted default on integer inputs; ragged M and N edges included
    M, N, K = 520, 488, 320
    _say("perm-off", dt, la, lb, no_perm)
    inp = _inputs_int(M, N, K, la, lb, dt, seed=71)
    from helpers import env
    with env(DGEMM_NO_PERM=no_perm):
        c0, i0 = run_gpu(inp, dt, "f32", split_k=1, force_tile="256x256")
    # the permuted in-register kernel (NT's and TT's defaults transpose with the LDS reads)
    with env(DGEMM_FORCE_DTL={("col", "row"): 0, ("row", "row"): 1}.get((la, lb))):
        c1, i1 = run_gpu(inp, dt, "f32", split_k=1, force_tile="256x256")
    assert i0["perm_block"] == 1 and i1["perm_block"] == 64
    assert i0["lds_pad_bytes"] == (0 if no_perm == 2 else 16)
    assert np.array_equal(c0, c1)
    _, ref = reference(inp, dt, "f32")
    assert np.array_equal(c0, ref)


@pytest.mark.parametrize("M,N,K", [(8, 8, 8), (8, 16, 64), (24, 40, 16)])
@pytest.mark.parametrize("la,lb", LAYOUTS)
def test_tiny_shapes(M, N, K, la, lb):
    _say("tiny", M, N, K, la, lb)
    inp = _inputs_int(M, N, K, la, lb, "f16", seed=81)
    c, _ = run_gpu(inp, "f16", "f32", split_k=1)
    _, ref = reference(inp, "f16", "f32")
    assert np.array_equal(c, ref)


DTL_LAYOUTS = [("row", "row"), ("row", "col"), ("col", "col")]   # a K-contiguous operand


def _dtl_bits(la, lb):
    return (1 if la == "row" else 0) | (2 if lb == "col" else 0)


@pytest.mark.parametrize("waves,sched,mfma", [(8, 1, 32), (8, 1, 16), (8, 0, 32), (4, 0, 32)])
@pytest.mark.parametrize("la,lb", DTL_LAYOUTS)
@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_direct_to_lds_integer_bit_exact(waves, sched, mfma, la, lb, fmt):
    # K-contiguous operands loaded straight into swizzled LDS rows, in the ping-pong (1) and
    # the pipeline (0) schedule, in 32x32x16 and (ping-pong) 16x16x32 blocks, the transposed
    # operand of NN and TT through the in-register transpose; ragged M, N and K (K = 200: the
    # last step has one 8-wide chunk) exercise the out-of-range zero fill
    M, N, K = 392 + 8, 648, 200
    _say("dtl-int", waves, sched, mfma, la, lb, fmt)
    inp = _inputs_int(M, N, K, la, lb, fmt, seed=91)
    from helpers import env
    with env(DGEMM_FORCE_DTL=1, DGEMM_FORCE_WAVES=waves, DGEMM_FORCE_SCHED=sched, DGEMM_FORCE_MFMA=mfma):
        c, info = run_gpu(inp, fmt, "f32", split_k=1, force_tile="256x256", guard=64)
    assert info["direct_lds"] == _dtl_bits(la, lb) and info["waves"] == waves
    assert info["mfma_m"] == mfma
    _, ref = reference(inp, fmt, "f32")
    assert np.array_equal(c, ref)


@pytest.mark.parametrize("mfma", [32, 16])
@pytest.mark.parametrize("la,lb", DTL_LAYOUTS)
def test_direct_to_lds_split_k_and_random(la, lb, mfma):
    from helpers import env
    M, N, K = 264, 520, 1032
    _say("dtl-split", la, lb, mfma)
    inp = _inputs_int(M, N, K, la, lb, "f16", seed=93)
    _, ref = reference(inp, "f16", "f32")
    with env(DGEMM_FORCE_DTL=1, DGEMM_FORCE_MFMA=mfma):
        for sk in (1, 4):
            c, info = run_gpu(inp, "f16", "f32", split_k=sk, force_tile="256x256", guard=16)
            assert info["direct_lds"] == _dtl_bits(la, lb) and info["split_k"] == sk
            assert info["mfma_m"] == mfma
            assert np.array_equal(c, ref), sk
        inp = _inputs_rand(520, 392, 328, la, lb, "bf16", seed=95)
        c, _ = run_gpu(inp, "bf16", "bf16", split_k=1, force_tile="256x256", guard=16)
    _, ref = reference(inp, "bf16", "bf16")
    amax, bmax = operand_max(inp, "bf16")
    check_tolerance(c, ref, "bf16", 328, amax, bmax, "dtl")


# Every selectable 256x256 main-loop variant: (schedule, direct-to-LDS, waves, block).
SCHED_VARIANTS = [(0, 0, 8, 32), (0, 0, 4, 32), (1, 0, 8, 32), (0, 1, 8, 32), (0, 1, 4, 32),
                  (1, 1, 8, 32), (0, 2, 8, 32), (1, 2, 8, 32), (2, 1, 4, 32), (2, 2, 4, 32),
                  (1, 1, 8, 16), (1, 2, 8, 16)]


@pytest.mark.parametrize("sched,dtl,waves,mfma", SCHED_VARIANTS)
@pytest.mark.parametrize("la,lb", LAYOUTS)
def test_every_schedule_variant_bit_exact(sched, dtl, waves, mfma, la, lb):
    if dtl == 1 and (la, lb) == ("col", "row"):
        pytest.skip("no K-contiguous operand to load directly")
    if dtl == 2 and (la, lb) == ("row", "col"):
        pytest.skip("no transposed operand")
    if sched == 2 and dtl == 1 and (la, lb) != ("row", "col"):
        pytest.skip("every operand direct: transposed ones with transposing reads (dtl 2)")
    from helpers import env
    M, N, K = 264, 520, 456
    _say("sched", sched, dtl, waves, mfma, la, lb)
    inp = _inputs_int(M, N, K, la, lb, "f16", seed=97)
    with env(DGEMM_FORCE_SCHED=sched, DGEMM_FORCE_DTL=dtl, DGEMM_FORCE_WAVES=waves,
             DGEMM_FORCE_MFMA=mfma):
        c, info = run_gpu(inp, "f16", "f32", split_k=1, force_tile="256x256", guard=16)
    assert info["waves"] == waves and info["schedule"] == sched and info["mfma_m"] == mfma
    assert (info["direct_lds"] != 0) == bool(dtl) and ((info["direct_lds"] & 12) != 0) == (dtl == 2)
    _, ref = reference(inp, "f16", "f32")
    assert np.array_equal(c, ref)


# The non-power-of-2 192x320 tile: (schedule, loader). Loader 0 = register-staged loads;
# 1 = K-contiguous operands straight into LDS; 2 = transposed operands too, in 64-wide K-row
# segments, transposed by the LDS reads. Schedule 1 is the 8-wave ping-pong with 16x16x32
# blocks (96x80 per wave), schedules 0 and 2 use 4 waves of 96x160 in 32x32x16 blocks.
NONPOW2 = [(1, 1), (1, 2), (0, 0), (0, 1), (0, 2), (2, 1), (2, 2)]


def _nonpow2_served(sched, dtl, la, lb):
    if dtl == 0:
        return True    # register-staged loads serve every layout
    if dtl == 1 and (la, lb) == ("col", "row"):
        return False   # no K-contiguous operand
    if dtl == 2 and (la, lb) == ("row", "col"):
        return False   # no transposed operand
    # schedules 1 and 2 load every operand straight into LDS: loader 1 serves TN only
    return not (sched in (1, 2) and dtl == 1 and (la, lb) != ("row", "col"))


def _nonpow2_bits(dtl, la, lb):
    if dtl == 0:
        return 0
    a_kc, b_kc = la == "row", lb == "col"
    bits = (1 if a_kc else 0) | (2 if b_kc else 0)
    if dtl == 2:
        bits |= (0 if a_kc else 4) | (0 if b_kc else 8)
    return bits


@pytest.mark.parametrize("sched,dtl", NONPOW2)
@pytest.mark.parametrize("la,lb", LAYOUTS)
@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_nonpow2_tile_direct_to_lds_bit_exact(sched, dtl, la, lb, fmt):
    # 192x320 tiles: two whole tiles and a ragged one in M (392 = 2 x 192 + 8) and in N
    # (648 = 2 x 320 + 8), 7 K steps and a ragged tail (456 = 7 x 64 + 8)
    if not _nonpow2_served(sched, dtl, la, lb):
        pytest.skip("this loader serves no operand of this layout pair on this schedule")
    from helpers import env
    M, N, K = 392, 648, 456
    _say("nonpow2", sched, dtl, la, lb, fmt)
    inp = _inputs_int(M, N, K, la, lb, fmt, seed=151 + dtl)
    with env(DGEMM_FORCE_SCHED=sched, DGEMM_FORCE_DTL=dtl):
        c, info = run_gpu(inp, fmt, "f32", split_k=1, force_tile="192x320", guard=64)
    assert (info["tile_m"], info["tile_n"], info["schedule"]) == (192, 320, sched)
    assert (info["waves"], info["mfma_m"]) == ((8, 16) if sched == 1 else (4, 32))
    assert info["direct_lds"] == _nonpow2_bits(dtl, la, lb)
    if dtl == 2:
        assert (info["perm_block"], info["perm_stride"], info["lds_pad_bytes"]) == (64, 8, 64)
    _, ref = reference(inp, fmt, "f32")
    assert np.array_equal(c, ref)


@pytest.mark.parametrize("la,lb", LAYOUTS)
def test_nonpow2_tile_direct_to_lds_split_k_and_random(la, lb):
    # the pipeline schedule with split-K (the partial tiles of 192 x 320 through the
    # fix-up), and random bf16 inputs to the acceptance bar on both schedules
    from helpers import env
    dtl = 1 if (la, lb) == ("row", "col") else 2
    M, N, K = 200, 328, 1032
    _say("nonpow2 split", la, lb, dtl)
    inp = _inputs_int(M, N, K, la, lb, "f16", seed=157)
    _, ref = reference(inp, "f16", "f32")
    for sched in (1, 0):
        with env(DGEMM_FORCE_SCHED=sched, DGEMM_FORCE_DTL=dtl):
            for sk in (1, 4):
                c, info = run_gpu(inp, "f16", "f32", split_k=sk, force_tile="192x320", guard=16)
                assert info["split_k"] == sk and info["direct_lds"] == _nonpow2_bits(dtl, la, lb)
                assert info["schedule"] == sched
                assert np.array_equal(c, ref), (sched, sk)
    inp = _inputs_rand(520, 392, 328, la, lb, "bf16", seed=159)
    _, ref = reference(inp, "bf16", "bf16")
    amax, bmax = operand_max(inp, "bf16")
    for sched in (1, 0, 2):
        with env(DGEMM_FORCE_SCHED=sched, DGEMM_FORCE_DTL=dtl):
            c, info = run_gpu(inp, "bf16", "bf16", split_k=1, force_tile="192x320", guard=16)
        assert info["schedule"] == sched
        check_tolerance(c, ref, "bf16", 328, amax, bmax, f"nonpow2 sched {sched}")


def _int4_group_inputs(M, N, K, group, seed):
    # codes U{0..15} packed along K, scales [K/group][N]; A = unit rows, so C rows are
    # dequantised weight rows exactly
    rng = np.random.default_rng(seed)
    q = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
    s = synth.to_bits(rng.uniform(0.005, 0.02, (K // group, N)), "f16")
    pick = rng.integers(0, K, size=M)
    a = np.zeros((M, K))
    a[np.arange(M), pick] = 1.0
    inp = {"M": M, "N": N, "K": K, "layout_a": "row", "layout_b": "col",
           "A": synth.store(synth.to_bits(a, "f16"), "row"), "B": synth.pack_u4_along_k(q),
           "scales": s.reshape(-1)}
    return inp, pick


@pytest.mark.parametrize("group,zero", [(32, 0), (64, 15), (256, 3), (1024, 8)])
@pytest.mark.parametrize("M,sk,tiled", [(16, 1, False), (16, 4, False), (5, 4, True),
                                        (300, 1, False), (300, 1, True)])
def test_int4_group_sizes_and_zero_points_bit_exact(group, zero, M, sk, tiled):
    # skinny (M <= 16) and tiled kernels, column-major and pre-tiled codes, split-K
    import dense_gemm_operand_amd as dg
    N, K = 320, 2048
    _say("int4 group/zero", group, zero, M, sk, tiled)
    inp, pick = _int4_group_inputs(M, N, K, group, seed=700 + group + zero + M)
    w = oracle.dequant_u4(inp["B"], inp["scales"], K, N, group=group, zero=zero)
    if tiled:
        inp = dict(inp, B=dg.gemm_pack_u4_tiled(inp["B"], N, K), layout_b="u4_tiled")
    c, info = run_gpu(inp, "f16", "f16", split_k=sk, int4=True, guard=16, group=group, zero=zero)
    assert info["kernel"] == (1 if M <= 16 else 0) and info["split_k"] == sk
    assert np.array_equal(oracle.decode(c, "f16"), w[pick])


@pytest.mark.parametrize("group,zero", [(32, 5), (512, 12)])
def test_int4_group_sizes_random_within_tolerance(group, zero):
    M, N, K = 384, 256, 1024
    rng = np.random.default_rng(710 + group)
    q = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
    s = synth.to_bits(rng.uniform(0.005, 0.02, (K // group, N)), "f16")
    a = synth.to_bits(rng.standard_normal((M, K)), "f16")
    inp = {"M": M, "N": N, "K": K, "layout_a": "row", "layout_b": "col",
           "A": synth.store(a, "row"), "B": synth.pack_u4_along_k(q), "scales": s.reshape(-1)}
    _say("int4 group random", group, zero)
    for sk, m in ((1, M), (0, 16)):
        sub = dict(inp, M=m, A=synth.store(a[:m], "row"))
        c, _ = run_gpu(sub, "f16", "f16", split_k=sk, int4=True, group=group, zero=zero)
        _, ref = reference(sub, "f16", "f16", int4=True, group=group, zero=zero)
        amax = float(np.abs(oracle.decode(a[:m].reshape(-1), "f16")).max())
        bmax = float(np.abs(oracle.dequant_u4(inp["B"], inp["scales"], K, N, group=group, zero=zero)).max())
        check_tolerance(c, ref, "f16", K, amax, bmax, f"int4 g{group} z{zero} M={m}")


INT4_SKINNY = ["2x8x2", "4x4x2", "2x8x4", "4x8x2"]   # the int4 default first


@pytest.mark.parametrize("v", INT4_SKINNY)
@pytest.mark.parametrize("sk", [1, 4])
def test_int4_skinny_variants_bit_exact(v, sk):
    # integer activations and power-of-two scales: every weight (q - 8) * s and every
    # partial sum is exact in fp32, so each variant must reproduce the oracle bit for bit;
    # M = 5 and N = 200 leave ragged rows and columns in every tile width
    from helpers import env
    M, N, K = 5, 200, 2048
    _say("int4-skinny", v, sk)
    inp = _int4_inputs(M, N, K, seed=65)
    rng = np.random.default_rng(66)
    inp["A"] = synth.store(synth.integer_matrix(rng, M, K, -2, 2, "f16"), "row")
    e = rng.integers(2, 7, size=(K // 128) * N)
    inp["scales"] = synth.to_bits(np.ldexp(1.0, -e), "f16").reshape(-1)
    with env(DGEMM_FORCE_SKINNY=v):
        c, info = run_gpu(inp, "f16", "f32", split_k=sk, int4=True, guard=8)
    assert info["kernel"] == 1 and info["split_k"] == sk
    assert (info["tile_n"], info["waves"]) == (16 * int(v.split("x")[0]), int(v.split("x")[1]))
    _, ref = reference(inp, "f16", "f32", int4=True)
    assert np.array_equal(c, ref)


FP16_SKINNY = ["4x4x2", "4x4x1", "4x8x2", "2x8x2"]


@pytest.mark.parametrize("v", FP16_SKINNY)
@pytest.mark.parametrize("M,N,K,sk", [(5, 200, 4104, 1), (16, 520, 8200, 4), (3, 64, 1000, 2)])
def test_fp16_skinny_variants_bit_exact(v, M, N, K, sk):
    # integer inputs: every partial sum is exact, so each variant (n-blocks x waves x
    # iterations per register set) must reproduce the oracle bit for bit, also with K not a
    # multiple of the wave iteration, ragged rows and columns, and split-K
    from helpers import env
    _say("fp16-skinny", v, M, N, K, sk)
    rng = np.random.default_rng(77)
    inp = {"M": M, "N": N, "K": K, "layout_a": "row", "layout_b": "col",
           "A": synth.store(synth.integer_matrix(rng, M, K, -3, 3, "f16"), "row"),
           "B": synth.store(synth.integer_matrix(rng, K, N, -3, 3, "f16"), "col")}
    with env(DGEMM_FORCE_SKINNY=v):
        c, info = run_gpu(inp, "f16", "f32", split_k=sk, guard=8)
    assert info["kernel"] == 1 and info["split_k"] == sk
    assert (info["tile_n"], info["waves"]) == (16 * int(v.split("x")[0]), int(v.split("x")[1]))
    _, ref = reference(inp, "f16", "f32")
    assert np.array_equal(c, ref)


TR_LAYOUTS = [("col", "col"), ("row", "row"), ("col", "row")]   # a transposed operand


def _tr_bits(la, lb):
    # direct_lds bits: 1/2 K-contiguous A/B loaded directly, 4/8 transposed A/B loaded
    # directly and transposed by the LDS reads
    return ((1 if la == "row" else 4) | (2 if lb == "col" else 8))


def _tr_sched_instantiated(fmt, la, lb, sched, mfma=32):
    # transposing reads: the pipeline (32x32x16) and the 16x16x32 ping-pong in every layout;
    # the 32x32x16 ping-pong in every layout for fp16, NT only for bf16
    return sched == 0 or mfma == 16 or fmt == "f16" or (la, lb) == ("col", "row")


# (schedule, matrix-core block): the 32x32x16 ping-pong and pipeline (two K rows per 1 KiB
# LDS block, B = 8, S = 4) and the 16x16x32 ping-pong (64-wide K-row segments, B = 64, S = 8)
TR_SCHED = [(1, 32), (0, 32), (1, 16)]
TR_PERM = {32: (8, 4, 64), 16: (64, 8, 64)}


@pytest.mark.parametrize("la,lb", TR_LAYOUTS)
@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("sched,mfma", TR_SCHED)
def test_transposing_lds_reads_integer_bit_exact(la, lb, fmt, sched, mfma):
    # transposed operands kept in global order in padded, K-row-permuted LDS blocks and
    # transposed by ds_read_b64_tr_b16, in the ping-pong (1) and the pipeline (0) schedule;
    # ragged M, N and K
    if not _tr_sched_instantiated(fmt, la, lb, sched, mfma):
        pytest.skip("not instantiated")
    from helpers import env
    M, N, K = 392 + 8, 648, 200
    _say("tr-int", la, lb, fmt, sched, mfma)
    inp = _inputs_int(M, N, K, la, lb, fmt, seed=101)
    with env(DGEMM_FORCE_DTL=2, DGEMM_FORCE_SCHED=sched, DGEMM_FORCE_MFMA=mfma):
        c, info = run_gpu(inp, fmt, "f32", split_k=1, force_tile="256x256", guard=64)
    assert info["direct_lds"] == _tr_bits(la, lb) and info["schedule"] == sched
    assert info["mfma_m"] == mfma
    assert (info["perm_block"], info["perm_stride"], info["lds_pad_bytes"]) == TR_PERM[mfma]
    _, ref = reference(inp, fmt, "f32")
    assert np.array_equal(c, ref)


@pytest.mark.parametrize("la,lb", TR_LAYOUTS)
@pytest.mark.parametrize("sched,mfma", TR_SCHED)
def test_transposing_lds_reads_split_k_and_random(la, lb, sched, mfma):
    from helpers import env
    M, N, K = 264, 520, 1032
    _say("tr-split", la, lb, sched, mfma)
    inp = _inputs_int(M, N, K, la, lb, "f16", seed=103)
    _, ref = reference(inp, "f16", "f32")
    with env(DGEMM_FORCE_DTL=2, DGEMM_FORCE_SCHED=sched, DGEMM_FORCE_MFMA=mfma):
        for sk in (1, 4):
            c, info = run_gpu(inp, "f16", "f32", split_k=sk, force_tile="256x256", guard=16)
            assert info["direct_lds"] == _tr_bits(la, lb) and info["split_k"] == sk
            assert info["schedule"] == sched and info["mfma_m"] == mfma
            assert np.array_equal(c, ref), sk
        fmt = "bf16" if _tr_sched_instantiated("bf16", la, lb, sched, mfma) else "f16"
        inp = _inputs_rand(520, 392, 328, la, lb, fmt, seed=105)
        c, info = run_gpu(inp, fmt, fmt, split_k=1, force_tile="256x256", guard=16)
        assert info["schedule"] == sched
    _, ref = reference(inp, fmt, fmt)
    amax, bmax = operand_max(inp, fmt)
    check_tolerance(c, ref, fmt, 328, amax, bmax, "tr")


@pytest.mark.parametrize("v,M", [("4x4x2", 5), ("2x8x4", 16), ("4x8x2", 5), ("2x8x2", 16), ("tile", 384)])
@pytest.mark.parametrize("sk", [1, 4])
def test_int4_tiled_layout_bit_exact(v, M, sk):
    # the same codes packed by gemm_pack_u4_tiled; the oracle reads the column-major packing.
    # Integer activations and power-of-two scales make every sum exact
    from helpers import env
    import dense_gemm_operand_amd as dg
    N, K = 192, 2048
    _say("int4-tiled", v, M, sk)
    inp = _int4_inputs(M, N, K, seed=131)
    rng = np.random.default_rng(132)
    inp["A"] = synth.store(synth.integer_matrix(rng, M, K, -2, 2, "f16"), "row")
    e = rng.integers(2, 7, size=(K // 128) * N)
    inp["scales"] = synth.to_bits(np.ldexp(1.0, -e), "f16").reshape(-1)
    _, ref = reference(inp, "f16", "f32", int4=True)
    tiled = dict(inp, B=dg.gemm_pack_u4_tiled(inp["B"], N, K), layout_b="u4_tiled")
    hooks = {"DGEMM_FORCE_SKINNY": v} if v != "tile" else {}
    with env(**hooks):
        c, info = run_gpu(tiled, "f16", "f32", split_k=sk, int4=True, guard=8)
    assert info["layout_b"] == dg.GEMM_U4_TILED and info["split_k"] == sk
    assert info["kernel"] == (0 if v == "tile" else 1)
    assert np.array_equal(c, ref)


@pytest.mark.parametrize("sched", [1, 0])
@pytest.mark.parametrize("tiled", [False, True])
@pytest.mark.parametrize("sk", [1, 4])
def test_int4_256_tiles_both_schedules_bit_exact(sched, tiled, sk):
    # row-major A on 256x256 tiles: the ping-pong schedule with A loaded straight into LDS
    # (1, the default) and the pipeline (0); ragged M and N, integer activations and
    # power-of-two scales, so every sum is exact
    from helpers import env
    import dense_gemm_operand_amd as dg
    M, N, K = 392, 384, 1152
    _say("int4-256", sched, tiled, sk)
    inp = _int4_inputs(M, N, K, seed=171)
    rng = np.random.default_rng(172)
    inp["A"] = synth.store(synth.integer_matrix(rng, M, K, -2, 2, "f16"), "row")
    e = rng.integers(2, 7, size=(K // 128) * N)
    inp["scales"] = synth.to_bits(np.ldexp(1.0, -e), "f16").reshape(-1)
    _, ref = reference(inp, "f16", "f32", int4=True)
    if tiled:
        inp = dict(inp, B=dg.gemm_pack_u4_tiled(inp["B"], N, K), layout_b="u4_tiled")
    with env(DGEMM_FORCE_SCHED=sched):
        c, info = run_gpu(inp, "f16", "f32", split_k=sk, int4=True, guard=16, force_tile="256x256")
    assert (info["tile_m"], info["split_k"]) == (256, sk)
    assert info["direct_lds"] == (1 if sched else 0)
    assert np.array_equal(c, ref)


@pytest.mark.parametrize("M,N,K", [(8, 8, 16), (24, 40, 8), (264, 8, 72), (8, 520, 136)])
@pytest.mark.parametrize("la,lb", LAYOUTS)
@pytest.mark.parametrize("dtl,sched", [(1, 1), (1, 0), (2, 1), (2, 0)])
def test_direct_to_lds_mostly_out_of_range_tiles(M, N, K, la, lb, dtl, sched):
    # one 256x256 tile almost entirely past M, N or K: the out-of-range direct-to-LDS loads
    # must leave zeros (or be ignored) and the partial steps must add nothing
    from helpers import env
    if dtl == 1 and (la, lb) == ("col", "row"):
        pytest.skip("no K-contiguous operand")
    if dtl == 2 and (la, lb) == ("row", "col"):
        pytest.skip("no transposed operand")
    _say("dtl-edge", M, N, K, la, lb, dtl, sched)
    inp = _inputs_int(M, N, K, la, lb, "f16", seed=151)
    with env(DGEMM_FORCE_DTL=dtl, DGEMM_FORCE_SCHED=sched):
        c, info = run_gpu(inp, "f16", "f32", split_k=1, force_tile="256x256", guard=32)
    assert info["direct_lds"] != 0 and info["schedule"] == sched
    _, ref = reference(inp, "f16", "f32")
    assert np.array_equal(c, ref)
