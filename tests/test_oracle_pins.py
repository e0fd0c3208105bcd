"""Pins of the CPU oracle against values that do not come from the oracle itself:
library conversions (numpy binary16/binary32, torch bfloat16), exact rational arithmetic,
closed-form products (identity, permutation, all-ones, Hadamard), hand-evaluated
fixtures under tests/golden/, and the page formulas' algebraic properties."""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from dense_gemm_operand_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
LAYOUTS = [("row", "row"), ("row", "col"), ("col", "row"), ("col", "col")]


# ---------------------------------------------------------------- format conversions

def test_decode_every_f16_pattern_matches_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.decode(bits, "f16")
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_decode_every_bf16_pattern_matches_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    ours = oracle.decode(bits, "bf16")
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def _hard_doubles(rng, n):
    """Doubles spread over many binades, plus exact ties, subnormal and overflow edges."""
    x = rng.standard_normal(n) * np.exp2(rng.integers(-30, 20, n))
    h = np.arange(0, 65504, 7, dtype=np.float64)
    ties = []
    for fmt_max in (65504.0,):
        ties += [fmt_max + 16.0, fmt_max + 15.999, 2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -24 * 1.5,
                 2.0 ** -14 - 2.0 ** -25, 1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11]
    return np.concatenate([x, -x, h, np.array(ties), -np.array(ties), [0.0, -0.0, np.inf, -np.inf]])


def test_encode_f16_matches_numpy_rne():
    rng = np.random.default_rng(7)
    x = _hard_doubles(rng, 200000)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.encode(x, "f16"), ref)


def test_encode_bf16_matches_torch_rne_on_float32_values():
    rng = np.random.default_rng(8)
    x32 = (rng.standard_normal(200000) * np.exp2(rng.integers(-120, 120, 200000))).astype(np.float32)
    # exact ties between two bfloat16 neighbours, both parities
    tie = (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x32 = np.concatenate([x32, tie, -tie])
    ref = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.encode(x32.astype(np.float64), "bf16"), ref)


def test_encode_f32_matches_numpy_cast():
    rng = np.random.default_rng(9)
    x = rng.standard_normal(200000) * np.exp2(rng.integers(-140, 120, 200000))
    ref = x.astype(np.float32).view(np.uint32)
    assert np.array_equal(oracle.encode(x, "f32"), ref)


# ---------------------------------------------------------------- layout map

def test_logical_map_hand_example():
    # logical [[1,2,3],[4,5,6]]: row-major stores 1..6, column-major stores 1,4,2,5,3,6
    want = np.array([[1, 2, 3], [4, 5, 6]], dtype=np.float64)
    assert np.array_equal(oracle.logical(np.arange(1, 7.0), 2, 3, "row"), want)
    assert np.array_equal(oracle.logical(np.array([1, 4, 2, 5, 3, 6.0]), 2, 3, "col"), want)


# ---------------------------------------------------------------- product

def _stored(bits_logical, layout):
    return synth.store(bits_logical, layout)


@pytest.mark.parametrize("la,lb", LAYOUTS)
def test_product_against_exact_rationals(la, lb):
    rng = np.random.default_rng(11)
    for M, N, K in [(1, 1, 1), (3, 5, 7), (8, 8, 8), (2, 7, 4)]:
        a = synth.to_bits(rng.uniform(-3, 3, (M, K)), "f16")
        b = synth.to_bits(rng.uniform(-3, 3, (K, N)), "f16")
        c64, _ = oracle.gemm(_stored(a, la), _stored(b, lb), M, N, K, la, lb, "f16", "f32")
        av = a.view(np.float16).astype(np.float64)
        bv = b.view(np.float16).astype(np.float64)
        for i in range(M):
            for j in range(N):
                exact = sum(Fraction(av[i, k]) * Fraction(bv[k, j]) for k in range(K))
                bound = K * 2.0 ** -53 * sum(abs(av[i, k] * bv[k, j]) for k in range(K))
                assert abs(Fraction(c64[i, j]) - exact) <= Fraction(bound)


@pytest.mark.parametrize("la,lb", LAYOUTS)
@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_identity_operands_reproduce_the_other(la, lb, fmt):
    rng = np.random.default_rng(12)
    n, m = 24, 40
    eye = synth.to_bits(np.eye(n), fmt)
    x = synth.integer_matrix(rng, n, m, -100, 100, fmt)
    _, c = oracle.gemm(_stored(eye, la), _stored(x, lb), n, m, n, la, lb, fmt, fmt)
    assert np.array_equal(c.reshape(n, m), x)          # I * X = X
    y = synth.integer_matrix(rng, m, n, -100, 100, fmt)
    _, c = oracle.gemm(_stored(y, la), _stored(eye, lb), m, n, n, la, lb, fmt, fmt)
    assert np.array_equal(c.reshape(m, n), y)          # Y * I = Y


@pytest.mark.parametrize("la,lb", LAYOUTS)
def test_permutation_matrix_permutes_rows(la, lb):
    rng = np.random.default_rng(13)
    n, m = 16, 24
    p = rng.permutation(n)
    P = np.zeros((n, n))
    P[np.arange(n), p] = 1.0                           # (P X)[i] = X[p[i]]
    x = synth.integer_matrix(rng, n, m, -50, 50, "f16")
    _, c = oracle.gemm(_stored(synth.to_bits(P, "f16"), la), _stored(x, lb), n, m, n, la, lb,
                       "f16", "f16")
    assert np.array_equal(c.reshape(n, m), x[p])


@pytest.mark.parametrize("la,lb", LAYOUTS)
def test_all_ones_gives_k(la, lb):
    M, N, K = 5, 16, 96
    a = synth.to_bits(np.ones((M, K)), "f16")
    b = synth.to_bits(np.ones((K, N)), "f16")
    c64, c = oracle.gemm(_stored(a, la), _stored(b, lb), M, N, K, la, lb, "f16", "f16")
    assert np.all(c64 == K)
    assert np.all(c == np.float16(K).view(np.uint16))


def _hadamard(n):
    h = np.array([[1.0]])
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


@pytest.mark.parametrize("K", [16, 64])
def test_hadamard_rows_are_orthogonal(K):
    H = _hadamard(K)
    a = synth.to_bits(H, "bf16")
    bt = synth.to_bits(H.T, "bf16")
    c64, _ = oracle.gemm(_stored(a, "col"), _stored(bt, "row"), K, K, K, "col", "row", "bf16", "f32")
    assert np.array_equal(c64, K * np.eye(K))


def test_nonsymmetric_product_catches_transposed_operand():
    # [[1,2],[3,4]] * [[5,6],[7,8]] = [[19,22],[43,50]] (hand computed)
    A = synth.to_bits(np.array([[1.0, 2], [3, 4]]), "f16")
    B = synth.to_bits(np.array([[5.0, 6], [7, 8]]), "f16")
    want = np.array([[19.0, 22], [43, 50]])
    for la, lb in LAYOUTS:
        c64, _ = oracle.gemm(_stored(A, la), _stored(B, lb), 2, 2, 2, la, lb, "f16", "f32")
        assert np.array_equal(c64, want)


def test_row_subset_equals_full_rows():
    rng = np.random.default_rng(14)
    a = rng.standard_normal((9, 13))
    b = rng.standard_normal((13, 6))
    assert np.array_equal(oracle.gemm_f64(a, b, (3, 7)), oracle.gemm_f64(a, b)[3:7])


def test_reduction_shapes_sum_exactly():
    # 4096 -> 1 and 4 x 4096 -> 4 sums (IREE PR 19596 test cases) as products with ones.
    x = np.arange(4 * 4096, dtype=np.float64).reshape(4, 4096) % 97 - 48
    ones = np.ones((4096, 1))
    assert oracle.gemm_f64(x[:1], ones)[0, 0] == x[0].sum()
    assert np.array_equal(oracle.gemm_f64(x, ones)[:, 0], x.sum(axis=1))


def test_output_rounding_is_single_rne():
    # product sums that land exactly between two binary16 neighbours round to even
    a = synth.to_bits(np.array([[1.0, 2.0 ** -11]]), "f16")      # 1 + 2^-11: tie
    b = synth.to_bits(np.array([[1.0], [1.0]]), "f16")
    _, c = oracle.gemm(a.reshape(-1), b.reshape(-1), 1, 1, 2, "row", "row", "f16", "f16")
    assert c[0, 0] == np.float16(1.0).view(np.uint16)
    a = synth.to_bits(np.array([[1.0 + 2.0 ** -10, 2.0 ** -11]]), "f16")  # odd + half ulp: up
    _, c = oracle.gemm(a.reshape(-1), b.reshape(-1), 1, 1, 2, "row", "row", "f16", "f16")
    assert c[0, 0] == np.float16(1.0 + 2.0 ** -9).view(np.uint16)


# ---------------------------------------------------------------- int4 dequant

def test_dequant_every_code_against_numpy_binary16_multiply():
    rng = np.random.default_rng(15)
    K, N = 256, 16
    q = np.tile(np.arange(16, dtype=np.uint8), (K * N) // 16).reshape(K, N)
    rng.shuffle(q.reshape(-1))
    s = synth.to_bits(rng.uniform(0.005, 0.02, (K // 128, N)), "f16")
    w = oracle.dequant_u4(synth.pack_u4_along_k(q), s.reshape(-1), K, N)
    sv = s.view(np.float16)
    # numpy's binary16 multiply rounds the exact product once
    ref = (q.astype(np.float16) - np.float16(8)) * sv[np.arange(K) // 128][:, :]
    assert np.array_equal(w, ref.astype(np.float64))
    # the expanded form q*s - 8*s is a different function (it rounds twice)
    two = (q.astype(np.float16) * sv[np.arange(K) // 128]) - (np.float16(8) * sv[np.arange(K) // 128])
    assert not np.array_equal(w, two.astype(np.float64))


@pytest.mark.parametrize("group,zero", [(32, 0), (64, 7), (256, 15), (512, 3)])
def test_dequant_other_groups_and_zero_points(group, zero):
    # (q - zero) * s[k // group][n] rounded once: numpy's binary16 subtract is exact here and
    # its multiply rounds once
    rng = np.random.default_rng(16 + group + zero)
    K, N = 1024, 8
    q = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
    s = synth.to_bits(rng.uniform(0.005, 0.02, (K // group, N)), "f16")
    w = oracle.dequant_u4(synth.pack_u4_along_k(q), s.reshape(-1), K, N, group=group, zero=zero)
    sv = s.view(np.float16)
    ref = (q.astype(np.float16) - np.float16(zero)) * sv[np.arange(K) // group]
    assert np.array_equal(w, ref.astype(np.float64))
    # scales laid out for another group size are refused
    if group != 128:
        with pytest.raises(AssertionError):
            oracle.dequant_u4(synth.pack_u4_along_k(q), s.reshape(-1), K, N, group=128, zero=zero)


def test_dequant_group_and_zero_hand_example():
    # K=64, N=1, group 32, zero 3: k=0 q=1 -> (1-3)*0.5; k=33 q=15 -> (15-3)*0.25
    K, N = 64, 1
    packed = np.full(K // 2, 0x33, dtype=np.uint8)     # q = 3 -> weight 0 elsewhere
    packed[0] = 0x31                                    # k=0 -> q=1, k=1 -> q=3
    packed[16] = 0xF3                                   # k=32 -> q=3, k=33 -> q=15
    s = synth.to_bits(np.array([[0.5], [0.25]]), "f16").reshape(-1)
    w = oracle.dequant_u4(packed, s, K, N, group=32, zero=3)[:, 0]
    assert w[0] == (1 - 3) * 0.5 and w[33] == (15 - 3) * 0.25
    assert np.count_nonzero(w) == 2


def test_dequant_nibble_order_and_scale_group_hand_example():
    # K=256, N=1: byte 0 = 0x21 -> q(k=0)=1, q(k=1)=2; scales 0.5 (k<128) and 0.25 (k>=128)
    K, N = 256, 1
    packed = np.full(K // 2, 0x88, dtype=np.uint8)     # q = 8 -> weight 0 everywhere else
    packed[0] = 0x21
    packed[64] = 0xF0                                   # k=128 -> q=0, k=129 -> q=15
    s = synth.to_bits(np.array([[0.5], [0.25]]), "f16").reshape(-1)
    w = oracle.dequant_u4(packed, s, K, N)[:, 0]
    assert w[0] == (1 - 8) * 0.5 and w[1] == (2 - 8) * 0.5
    assert w[128] == (0 - 8) * 0.25 and w[129] == (15 - 8) * 0.25
    assert np.count_nonzero(w) == 4


def test_int4_gemm_identity_rows_return_dequantized_weights():
    rng = np.random.default_rng(16)
    K, N = 256, 24
    q = rng.integers(0, 16, (K, N)).astype(np.uint8)
    s = synth.to_bits(rng.uniform(0.005, 0.02, (K // 128, N)), "f16").reshape(-1)
    eye = synth.to_bits(np.eye(K), "f16")
    _, c = oracle.gemm(eye.reshape(-1), synth.pack_u4_along_k(q), K, N, K, "row", "col", "f16",
                       "f16", scales_bits=s)
    w = oracle.dequant_u4(synth.pack_u4_along_k(q), s, K, N)
    assert np.array_equal(oracle.decode(c, "f16"), w)


# ---------------------------------------------------------------- host rules from the pages

def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.strip() for ln in f if ln.strip() and not ln.startswith("#")]


def test_perm_fwd_hand_examples():
    for ln in _golden("perm_examples.txt"):
        head, vals = ln.split("|")
        B, S = map(int, head.split())
        assert [oracle.perm_fwd(i, B, S) for i in range(B)] == list(map(int, vals.split()))


def test_perm_is_bijection_and_inverse_round_trips_exhaustively():
    for B in range(1, 513):
        for S in range(1, B + 1):
            if B % S:
                continue
            f = [oracle.perm_fwd(i, B, S) for i in range(B)]
            assert sorted(f) == list(range(B))
            assert all(oracle.perm_inv(f[i], B, S) == i for i in range(B))


def test_perm_without_divisibility_is_not_a_bijection():
    # B=10, S=4 maps two indices onto 4: the planner must only pick S | B
    f = [oracle.perm_fwd(i, 10, 4) for i in range(10)]
    assert len(set(f)) < 10


def test_splitk_factor_hand_cases():
    for ln in _golden("splitk_cases.txt"):
        lhs, want = ln.split("->")
        cus, M, N, K, bm, bn, bk = map(int, lhs.split())
        assert oracle.splitk_factor(M, N, K, bm, bn, bk, cus) == int(want), ln


def test_fp8_e4m3_decode_matches_torch_for_every_code():
    # all 256 byte patterns against torch's float8_e4m3fn (OCP E4M3) conversion
    import torch
    codes = np.arange(256, dtype=np.uint8)
    v = oracle.decode(codes, "f8")
    t = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(v), np.isnan(t))
    assert np.array_equal(v[~np.isnan(v)], t[~np.isnan(t)])
    assert np.array_equal(np.signbit(v[~np.isnan(v)]), np.signbit(t[~np.isnan(t)]))


def test_fp8_e4m3_closed_form_values():
    v = oracle.decode(np.arange(256, dtype=np.uint8), "f8")
    assert v[0x38] == 1.0 and v[0xB8] == -1.0 and v[0x40] == 2.0 and v[0xC0] == -2.0
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0               # largest finite
    assert v[0x77] == 240.0 and v[0x30] == 0.5 and v[0x3C] == 1.5
    assert v[0x08] == 2.0 ** -6 and v[0x01] == 2.0 ** -9        # smallest normal, subnormal
    assert v[0x00] == 0.0 and not np.signbit(v[0x00]) and np.signbit(v[0x80])
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF]) and np.isnan(v).sum() == 2
    assert len(set(v[~np.isnan(v)].tolist())) == 253            # +0 and -0 compare equal
    pos = v[0x00:0x7F]
    assert np.all(np.diff(pos) > 0)                             # codes ordered by value
    # integers 0..16 are exact
    for i in range(17):
        assert i in set(pos.tolist())


def test_fp8_gemm_with_integer_entries_is_the_integer_product():
    rng = np.random.default_rng(9)
    M, N, K = 5, 7, 33
    ai = rng.integers(-8, 9, size=(M, K))
    bi = rng.integers(-8, 9, size=(K, N))
    for la in ("row", "col"):
        for lb in ("row", "col"):
            a = synth.to_bits(ai.astype(np.float64), "f8")
            b = synth.to_bits(bi.astype(np.float64), "f8")
            c64, _ = oracle.gemm(synth.store(a, la), synth.store(b, lb), M, N, K, la, lb,
                                 "f8", "f32")
            assert np.array_equal(c64, (ai @ bi).astype(np.float64))


# ---------------------------------------------------------------- attention (P * V)

def _att(q, k, v, scale):
    return oracle.attention_f64(q[None], k[None], v[None], scale)[0]


def test_attention_zero_queries_average_the_values():
    # q = 0: every score is 0, the weights are uniform, each output row is the mean of V
    rng = np.random.default_rng(301)
    Sk, D = 37, 16
    k = rng.standard_normal((Sk, D))
    v = rng.standard_normal((Sk, D))
    o = _att(np.zeros((5, D)), k, v, 0.3)
    assert np.allclose(o, np.broadcast_to(v.mean(axis=0), o.shape), rtol=0, atol=1e-15)


def test_attention_single_key_returns_its_value_exactly():
    rng = np.random.default_rng(302)
    q, k, v = rng.standard_normal((4, 8)), rng.standard_normal((1, 8)), rng.standard_normal((1, 8))
    assert np.array_equal(_att(q, k, v, 2.0), np.broadcast_to(v[0], (4, 8)))


def test_attention_two_keys_closed_form():
    # q = (2, 0, 0), k0 = (1, 0, 0), k1 = (0, 1, 0), scale 0.5: scores 1 and 0, so the
    # weight of key 0 is the logistic function at 1 = e / (1 + e) = 0.7310585786300049
    q = np.array([[2.0, 0.0, 0.0]])
    k = np.array([[1.0, 0.0, 0.0], [0.0, 1.0, 0.0]])
    v = np.array([[1.0, 10.0, -3.0], [0.0, -2.0, 5.0]])
    w0 = 0.7310585786300049
    want = w0 * v[0] + (1.0 - w0) * v[1]
    assert np.allclose(_att(q, k, v, 0.5)[0], want, rtol=1e-15, atol=1e-15)
    # swapping the roles of the keys swaps the weights (the query side is not transposed)
    assert np.allclose(_att(q, k[::-1].copy(), v, 0.5)[0], (1 - w0) * v[0] + w0 * v[1], rtol=1e-15, atol=1e-15)


def test_attention_dominant_key_selects_its_value():
    # one key scores 200 above the others: its weight is 1 to within exp(-200)
    rng = np.random.default_rng(303)
    Sk, D = 50, 8
    k = rng.standard_normal((Sk, D)) * 0.01
    q = np.zeros((3, D))
    q[:, 0] = 1.0
    k[17, 0] = 200.0
    v = rng.standard_normal((Sk, D))
    assert np.allclose(_att(q, k, v, 1.0), np.broadcast_to(v[17], (3, D)), rtol=0, atol=1e-12)


def test_attention_invariances():
    rng = np.random.default_rng(304)
    Sq, Sk, D = 6, 23, 12
    q, k, v = rng.standard_normal((Sq, D)), rng.standard_normal((Sk, D)), rng.standard_normal((Sk, D))
    o = _att(q, k, v, 0.7)
    # a vector added to every key shifts each query's scores by a constant: no change
    c = rng.standard_normal(D)
    assert np.allclose(_att(q, k + c, v, 0.7), o, rtol=1e-12, atol=1e-12)
    # keys and values permuted together: no change; queries permuted: rows permuted
    pk = rng.permutation(Sk)
    assert np.allclose(_att(q, k[pk], v[pk], 0.7), o, rtol=1e-12, atol=1e-13)
    pq = rng.permutation(Sq)
    assert np.allclose(_att(q[pq], k, v, 0.7), o[pq], rtol=0, atol=1e-15)
    # the scale multiplies the scores: scale s on q equals scale 1 on s*q
    assert np.allclose(_att(0.7 * q, k, v, 1.0), o, rtol=1e-12, atol=1e-13)
    # linear in V, and every output lies in the convex hull of the value rows
    v2 = rng.standard_normal((Sk, D))
    assert np.allclose(_att(q, k, 2 * v - 3 * v2, 0.7), 2 * o - 3 * _att(q, k, v2, 0.7), rtol=1e-12, atol=1e-12)
    assert np.all(o <= v.max(axis=0) + 1e-15) and np.all(o >= v.min(axis=0) - 1e-15)


def test_attention_slices_are_independent_and_rows_sample_correctly():
    rng = np.random.default_rng(305)
    BH, Sq, Sk, D = 3, 5, 9, 4
    q, k, v = (rng.standard_normal((BH, Sq, D)), rng.standard_normal((BH, Sk, D)),
               rng.standard_normal((BH, Sk, D)))
    o = oracle.attention_f64(q, k, v, 0.5)
    for h in range(BH):
        assert np.array_equal(o[h], _att(q[h], k[h], v[h], 0.5))
    part = oracle.attention_f64(q, k, v, 0.5, rows=(4, 12))
    assert np.array_equal(part, o.reshape(-1, D)[4:12])


def test_attention_from_bits_rounds_once():
    # fp16 bits in, fp16 bits out: the result is the fp64 value rounded by numpy
    rng = np.random.default_rng(306)
    BH, Sq, Sk, D = 2, 4, 7, 8
    qb = synth.to_bits(rng.standard_normal((BH, Sq, D)), "f16")
    kb = synth.to_bits(rng.standard_normal((BH, Sk, D)), "f16")
    vb = synth.to_bits(rng.standard_normal((BH, Sk, D)), "f16")
    o64, obits = oracle.attention(qb, kb, vb, BH, Sq, Sk, D, "f16", "f16", 0.25)
    assert np.array_equal(obits.reshape(-1), o64.reshape(-1).astype(np.float16).view(np.uint16))
