"""GPU parity of the attention forward (include/dattn.h) against the CPU oracle.

Bar, derived from the arithmetic: P is rounded once to the operand format before P * V and
O once to the output format, each a relative error of at most u (u = 2^-11 for fp16,
2^-8 for bf16), and fp32 sums over Sk keys add at most Sk * 2^-24 relative; so every
element is within (2u + Sk * 2^-24) * max|v| of the exact value, and the relative
Frobenius error is at most 2u. Exact cases: with zero queries every weight is exactly 1
(P = 1 in any format), so integer V and a power-of-two Sk give the exact mean; with
one-hot scores (every other key 64 below, its weight rounds to 0) each output row is
exactly one value row."""
import numpy as np
import pytest

import oracle
from dense_gemm_operand_amd import synth

pytestmark = pytest.mark.gpu

U = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}


def _say(*a):
    print("[case]", *a, flush=True)


def run_attn(inp: dict, guard: int = 64):
    """O bits (uint16, [BH][Sq][D]) from the HIP kernel through the C ABI."""
    import torch
    import dense_gemm_operand_amd as dg
    BH, Sq, Sk, D = inp["BH"], inp["Sq"], inp["Sk"], inp["D"]
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda()
    Q, K, V = dev(inp["Q"]), dev(inp["K"]), dev(inp["V"])
    n = BH * Sq * D
    O = torch.full((n + guard,), 0x5A5A, dtype=torch.int16, device="cuda")
    dg.attn_fwd(Q, K, V, O, BH, Sq, Sk, D, inp["dtype"], inp["scale"])
    torch.cuda.synchronize()
    out = O.cpu().numpy().view(np.uint16)
    assert np.all(out[n:] == 0x5A5A), "write past the end of O"
    return out[:n].reshape(BH, Sq, D)


def _inputs(BH, Sq, Sk, dtype, seed, D=128):
    w = synth.ATTN_WORKLOADS["attn_4096"]
    return synth.make_attn_inputs(w, BH=BH, Sq=Sq, Sk=Sk, dtype=dtype, seed=seed)


def check_bar(o_bits, inp, rows=None, what=""):
    BH, Sq, Sk, D, dt = inp["BH"], inp["Sq"], inp["Sk"], inp["D"], inp["dtype"]
    o64, _ = oracle.attention(inp["Q"], inp["K"], inp["V"], BH, Sq, Sk, D, dt, dt, inp["scale"], rows=rows)
    g = oracle.decode(np.ascontiguousarray(o_bits).reshape(-1), dt).reshape(o64.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    vmax = float(np.abs(oracle.decode(inp["V"], dt)).max())
    u = U[dt]
    err = np.abs(g - o64)
    bound = (2 * u + Sk * 2.0 ** -24) * vmax
    assert err.max() <= bound, f"{what}: max error {err.max():.3e} > {bound:.3e}"
    rel = np.linalg.norm(g - o64) / np.linalg.norm(o64)
    assert rel <= 2 * u, f"{what}: relative Frobenius error {rel:.3e} > {2 * u:.3e}"
    # reported beside the bar: the same error against the oracle rounded once to the output
    # format, the reference the GEMM's tolerance uses
    r = oracle.decode(oracle.encode(o64, dt), dt)
    rel_r = np.linalg.norm(g - r) / np.linalg.norm(r)
    _say(f"  {what}: relative Frobenius error {rel:.3e} against the exact output (bar {2 * u:.3e}), "
         f"{rel_r:.3e} against the output rounded to {dt}")
    return rel, float(err.max())


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("BH,Sq,Sk", [(2, 256, 128), (3, 300, 200), (1, 512, 640), (2, 17, 1),
                                      (1, 1, 333), (2, 260, 129)])
def test_attention_random_within_bar(BH, Sq, Sk, dtype):
    # several query blocks and key tiles, ragged in both (masked keys, unstored rows)
    _say("attn rand", BH, Sq, Sk, dtype)
    inp = _inputs(BH, Sq, Sk, dtype, seed=401 + Sq + Sk)
    o = run_attn(inp)
    check_bar(o, inp, what=f"{BH}x{Sq}x{Sk} {dtype}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("Sk", [64, 128, 256, 1024])
def test_attention_zero_queries_exact_mean(Sk, dtype):
    # every score is 0, every weight exactly 1: O = sum(v) / Sk exactly for integer V
    BH, Sq, D = 2, 300, 128
    rng = np.random.default_rng(411)
    inp = {"BH": BH, "Sq": Sq, "Sk": Sk, "D": D, "dtype": dtype, "scale": 0.125,
           "Q": synth.to_bits(np.zeros((BH, Sq, D)), dtype).reshape(-1),
           "K": synth.to_bits(rng.standard_normal((BH, Sk, D)), dtype).reshape(-1),
           "V": synth.to_bits(rng.integers(-8, 9, size=(BH, Sk, D)).astype(np.float64), dtype).reshape(-1)}
    _say("attn mean", Sk, dtype)
    o = run_attn(inp)
    _, ref = oracle.attention(inp["Q"], inp["K"], inp["V"], BH, Sq, Sk, D, dtype, dtype, inp["scale"])
    assert np.array_equal(o, ref.reshape(o.shape))


def _one_hot_inputs(BH, Sq, Sk, dtype, seed):
    # key pos[c] owns channel c (K = 0 there, -8 on every other channel of that key; every
    # other key is -8 everywhere); query i is 8 on channel c_i and 0 elsewhere; scale 1:
    # the owner of c_i scores 0 and every other key -64, whose weight exp(-64) rounds to 0
    D = 128
    rng = np.random.default_rng(seed)
    k = np.full((BH, Sk, D), -8.0)
    q = np.zeros((BH, Sq, D))
    want_key = np.zeros((BH, Sq), dtype=np.int64)
    nch = min(D, Sk)
    for h in range(BH):
        pos = rng.choice(Sk, size=nch, replace=False)
        k[h, pos, np.arange(nch)] = 0.0
        c = rng.integers(0, nch, size=Sq)
        q[h, np.arange(Sq), c] = 8.0
        want_key[h] = pos[c]
    v = rng.standard_normal((BH, Sk, D))
    inp = {"BH": BH, "Sq": Sq, "Sk": Sk, "D": D, "dtype": dtype, "scale": 1.0,
           "Q": synth.to_bits(q, dtype).reshape(-1), "K": synth.to_bits(k, dtype).reshape(-1),
           "V": synth.to_bits(v, dtype).reshape(-1)}
    vb = inp["V"].reshape(BH, Sk, D)
    want = np.stack([vb[h, want_key[h]] for h in range(BH)])
    return inp, want


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("BH,Sq,Sk", [(2, 512, 384), (1, 300, 200), (3, 64, 130)])
def test_attention_one_hot_selects_value_rows_exactly(BH, Sq, Sk, dtype):
    _say("attn one-hot", BH, Sq, Sk, dtype)
    inp, want = _one_hot_inputs(BH, Sq, Sk, dtype, seed=421 + Sk)
    o = run_attn(inp)
    assert np.array_equal(o, want)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_attention_many_tiny_weights(dtype):
    # one key scores 0, the other 4095 score -16 ln 2: their weights 2^-16 are subnormal
    # in fp16 and together carry 1/17 of the mass, so flushing them (in the weights' row sum
    # or in the matrix product) would miss the bar by far
    BH, Sq, Sk, D = 2, 64, 4096, 128
    rng = np.random.default_rng(441)
    q = np.zeros((BH, Sq, D))
    q[:, :, 0] = 1.0
    k = np.zeros((BH, Sk, D))
    k[:, :, 0] = -16.0 * np.log(2.0)
    k[:, 100, 0] = 0.0
    inp = {"BH": BH, "Sq": Sq, "Sk": Sk, "D": D, "dtype": dtype, "scale": 1.0,
           "Q": synth.to_bits(q, dtype).reshape(-1), "K": synth.to_bits(k, dtype).reshape(-1),
           "V": synth.to_bits(rng.standard_normal((BH, Sk, D)), dtype).reshape(-1)}
    _say("attn tiny weights", dtype)
    check_bar(run_attn(inp), inp, what=f"tiny weights {dtype}")


@pytest.mark.parametrize("scale", [-0.0883883476, 0.0])
def test_attention_negative_and_zero_scale(scale):
    # a negative scale turns the smallest score into the largest weight; a zero scale
    # gives every key the same weight (the plain mean), also with a ragged last unit
    _say("attn scale", scale)
    inp = _inputs(2, 200, 333, "f16", seed=451)
    inp["scale"] = scale
    check_bar(run_attn(inp), inp, what=f"scale {scale}")


def test_attention_full_size_sampled_rows():
    # the bench's workload (batch 4 x 16 heads, 4096 x 4096, head dim 128, fp16): rows of
    # the first, a middle and the last slice, at the start, middle and end of the sequence
    w = synth.ATTN_WORKLOADS["attn_4096"]
    inp = synth.make_attn_inputs(w)
    _say("attn full")
    o = run_attn(inp, guard=16).reshape(-1, inp["D"])
    Sq = inp["Sq"]
    for h in (0, 31, inp["BH"] - 1):
        for r0 in (0, 2044, Sq - 8):
            rows = (h * Sq + r0, h * Sq + r0 + 8)
            check_bar(o[rows[0]:rows[1]], inp, rows=rows, what=f"full slice {h} rows {r0}")


def test_attention_full_size_one_hot_every_element():
    _say("attn full one-hot")
    inp, want = _one_hot_inputs(64, 4096, 4096, "f16", seed=431)
    o = run_attn(inp, guard=16)
    assert np.array_equal(o, want)
