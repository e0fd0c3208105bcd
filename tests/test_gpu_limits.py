"""GPU runs at the largest operand sizes the library accepts (every operand below 2 GiB, the
limit of its 32-bit buffer offsets), checked on every output element by properties that
hold exactly at any size:
  * A made of unit rows picks whole rows of B: C[i, :] = B[pick[i], :] exactly (one nonzero
    product per sum), so the largest byte offsets of B are read and checked;
  * attention with zero queries weighs every key exactly 1, so O is the exact mean of V
    (values 0/1, 2^22 keys: every sum is an integer below 2^24, the division a power of two).
"""
import numpy as np
import pytest

import oracle
from dense_gemm_operand_amd import synth

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)


def _small_int_bits(rng, shape, lo, hi, fmt):
    # integers in [lo, hi] as storage bits via a table (the arrays are too large for fp64)
    vals = np.arange(lo, hi + 1, dtype=np.float64)
    table = synth.to_bits(vals, fmt)
    return table[rng.integers(0, hi - lo + 1, size=shape, dtype=np.uint8)]


def _unit_rows(rng, M, K, fmt):
    pick = rng.integers(0, K, size=M)
    a = np.zeros((M, K))
    a[np.arange(M), pick] = 1.0
    return synth.to_bits(a, fmt), pick


def _run_unit_rows(M, N, K, la, fmt, seed):
    import torch
    import dense_gemm_operand_amd as dg
    rng = np.random.default_rng(seed)
    # B column-major (K-contiguous): stored [N][K]
    b_nk = _small_int_bits(rng, (N, K), -8, 8, fmt)
    a_bits, pick = _unit_rows(rng, M, K, fmt)
    A = synth.store(a_bits, la)
    plan = dg.gemm_plan(M, N, K, la, "col", fmt, fmt, "f32", 1)
    try:
        info = dg.gemm_plan_query(plan)
        dev = (lambda x: torch.from_numpy(x.view(np.int16)).cuda()) if fmt != "f8" else \
              (lambda x: torch.from_numpy(x).cuda())
        dA, dB = dev(np.ascontiguousarray(A)), dev(b_nk.reshape(-1))
        C = torch.empty(M * N, dtype=torch.int32, device="cuda")
        dg.gemm_run(plan, dA, dB, None, C)
        torch.cuda.synchronize()
        got = oracle.decode(C.cpu().numpy().view(np.uint32), "f32").reshape(M, N)
    finally:
        dg.gemm_plan_destroy(plan)
    want = oracle.decode(np.ascontiguousarray(b_nk[:, pick].T).reshape(-1), fmt).reshape(M, N)
    return got, want, info


@pytest.mark.parametrize("M,la", [(16, "row"), (512, "col")])
def test_fp16_b_just_below_2_gib(M, la):
    # B: 32768 x 32760 fp16 = 2 146 959 360 bytes (the limit is 2^31 - 16)
    N, K = 32768, 32760
    _say("limit fp16", M, la, N, K)
    got, want, info = _run_unit_rows(M, N, K, la, "f16", seed=801 + M)
    assert info["kernel"] == (1 if M <= 16 else 0)
    assert np.array_equal(got, want)


def test_fp8_b_just_below_2_gib():
    # B: 65536 x 32752 fp8 = 2 146 435 072 bytes
    M, N, K = 256, 65536, 32752
    _say("limit fp8", M, N, K)
    got, want, _ = _run_unit_rows(M, N, K, "col", "f8", seed=811)
    assert np.array_equal(got, want)


def test_attention_2_pow_22_keys():
    # K, V: 1 slice x 2^22 keys x 128 = 2^30 bytes each; zero queries -> O = mean of V exactly
    import torch
    import dense_gemm_operand_amd as dg
    BH, Sq, Sk, D = 1, 300, 1 << 22, 128
    _say("limit attention", BH, Sq, Sk)
    rng = np.random.default_rng(821)
    v01 = rng.integers(0, 2, size=(Sk, D), dtype=np.uint8)
    vbits = synth.to_bits(np.array([0.0, 1.0]), "f16")[v01]
    kbits = _small_int_bits(rng, (Sk, D), -2, 2, "f16")
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x).reshape(-1).view(np.int16)).cuda()
    Q = torch.zeros(BH * Sq * D, dtype=torch.int16, device="cuda")
    O = torch.empty(BH * Sq * D, dtype=torch.int16, device="cuda")
    dg.attn_fwd(Q, dev(kbits), dev(vbits), O, BH, Sq, Sk, D, "f16", 0.0883883476)
    torch.cuda.synchronize()
    got = oracle.decode(O.cpu().numpy().view(np.uint16), "f16").reshape(Sq, D)
    mean = v01.sum(axis=0, dtype=np.int64).astype(np.float64) / Sk
    want = oracle.decode(oracle.encode(mean, "f16"), "f16")
    assert np.array_equal(got, np.broadcast_to(want, got.shape))
