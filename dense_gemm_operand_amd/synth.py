"""Seeded synthetic inputs for the operand-layout GEMM workloads.

This module only draws random numbers and lays them out in memory; it holds none of the
product's arithmetic. Both the HIP path's tests/benchmark and the CPU oracle consume the
same bytes it produces.

Recipe (one PCG64 generator per workload, seed 1234 + workload index; values drawn in
fp64 in the order A, B, codes, scales, then converted once to the storage format):
  square_tt_256     256^3 fp16, A row-major, B row-major, U[-1, 1], fp32 C
  square_4096       4096^3 fp16, one logical A and B, N(0,1)/sqrt(K), fp16 C, any layouts
  nonpow2_bf16      M=3072 N=5120 K=6144 bf16, A col-major, B row-major, N(0, 0.02), bf16 C
  skinny_splitk     M=16 N=8192 K=28672 fp16, A row-major, B col-major, U[-0.5, 0.5], fp16 C
  int4_m16/int4_m4096  M x 8192 x 8192, A fp16 row-major N(0,1); B 4-bit codes U{0..15}
                    packed two per byte along K (low nibble = even k), zero point 8,
                    fp16 scales [K/128][N] U[0.005, 0.02]; fp16 C
  square_4096_f8    4096^3 8-bit E4M3 (OCP) operands, BLAS NN storage, N(0, 1), fp16 C
Attention forward (Q, K, V and O [batch*heads][seq][head dim], head dim contiguous; drawn
in the order Q, K, V, each N(0, 1), converted once; scale 1/sqrt(head dim)):
  attn_4096         batch 4 x 16 heads, 4096 queries and keys, head dim 128, fp16
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    index: int
    M: int
    N: int
    K: int
    layout_a: str          # "row" or "col" storage of the logical M x K operand
    layout_b: str          # "row" or "col" storage of the logical K x N operand
    dtype_ab: str          # "f16" or "bf16" (A; B too unless int4)
    dtype_c: str           # "f32", "f16" or "bf16"
    dist: str              # "uniform1", "normal_sqrtk", "normal002", "uniform05", "int4"
    int4: bool = False
    split_k: int = 0       # 0 = let the planner choose
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    "square_tt_256": Workload("square_tt_256", 0, 256, 256, 256, "row", "row", "f16", "f32",
                              "uniform1", split_k=1),
    "square_4096": Workload("square_4096", 1, 4096, 4096, 4096, "col", "col", "f16", "f16",
                            "normal_sqrtk", split_k=1),
    "nonpow2_bf16": Workload("nonpow2_bf16", 2, 3072, 5120, 6144, "col", "row", "bf16", "bf16",
                             "normal002", split_k=1),
    "skinny_splitk": Workload("skinny_splitk", 3, 16, 8192, 28672, "row", "col", "f16", "f16",
                              "uniform05"),
    "int4_m16": Workload("int4_m16", 4, 16, 8192, 8192, "row", "col", "f16", "f16", "int4",
                         int4=True),
    "int4_m4096": Workload("int4_m4096", 4, 4096, 8192, 8192, "row", "col", "f16", "f16", "int4",
                           int4=True, split_k=1),
    "square_4096_f8": Workload("square_4096_f8", 5, 4096, 4096, 4096, "col", "col", "f8", "f16",
                               "normal1", split_k=1),
}

LAYOUT_LETTERS = {  # BLAS column-major lettering -> (A storage, B storage)
    "NN": ("col", "col"), "NT": ("col", "row"), "TN": ("row", "col"), "TT": ("row", "row"),
}


@dataclass(frozen=True)
class AttnWorkload:
    name: str
    index: int
    batch: int
    heads: int
    seq_q: int
    seq_k: int
    head_dim: int
    dtype: str             # "f16" or "bf16" (Q, K, V and O)

    @property
    def BH(self) -> int:
        return self.batch * self.heads


ATTN_WORKLOADS = {
    "attn_4096": AttnWorkload("attn_4096", 6, 4, 16, 4096, 4096, 128, "f16"),
}


def make_attn_inputs(w: AttnWorkload, BH: int | None = None, Sq: int | None = None,
                     Sk: int | None = None, dtype: str | None = None,
                     seed: int | None = None) -> dict:
    """Seeded Q, K, V bits ([BH][S][D], flat) of an attention workload, optionally resized."""
    BH = w.BH if BH is None else BH
    Sq = w.seq_q if Sq is None else Sq
    Sk = w.seq_k if Sk is None else Sk
    dt = w.dtype if dtype is None else dtype
    D = w.head_dim
    rng = np.random.default_rng(1234 + w.index if seed is None else seed)
    q = to_bits(rng.standard_normal((BH, Sq, D)), dt)
    k = to_bits(rng.standard_normal((BH, Sk, D)), dt)
    v = to_bits(rng.standard_normal((BH, Sk, D)), dt)
    return {"BH": BH, "Sq": Sq, "Sk": Sk, "D": D, "dtype": dt, "scale": 1.0 / np.sqrt(D),
            "Q": q.reshape(-1), "K": k.reshape(-1), "V": v.reshape(-1)}


def to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """fp64 -> storage bits (uint16 for f16/bf16, uint8 for f8) with the library
    conversions of numpy (binary16) and torch (bfloat16, and float8_e4m3fn for f8: the
    E4M3 format in the OCP convention)."""
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    if dtype == "f8":
        import torch
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.float8_e4m3fn)
        return t.view(torch.uint8).numpy()
    if dtype == "bf16":
        import torch
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16)
    raise ValueError(dtype)


def store(logical_bits: np.ndarray, layout: str) -> np.ndarray:
    """Flat storage of a logical (rows x cols) matrix: row-major keeps the order,
    column-major stores element (r, c) at r + c * rows."""
    if layout == "row":
        return np.ascontiguousarray(logical_bits).reshape(-1)
    return np.ascontiguousarray(logical_bits.T).reshape(-1)


def pack_u4_along_k(q_kn: np.ndarray) -> np.ndarray:
    """Pack K x N codes (0..15) two per byte along K: byte n*K/2 + k/2, low nibble even k."""
    K, N = q_kn.shape
    qt = np.ascontiguousarray(q_kn.T.astype(np.uint8))       # N x K
    return (qt[:, 0::2] | (qt[:, 1::2] << 4)).reshape(-1)


def _draw(rng: np.random.Generator, dist: str, shape, K: int) -> np.ndarray:
    if dist == "uniform1":
        return rng.uniform(-1.0, 1.0, size=shape)
    if dist == "normal_sqrtk":
        return rng.standard_normal(size=shape) / np.sqrt(K)
    if dist == "normal002":
        return rng.normal(0.0, 0.02, size=shape)
    if dist == "uniform05":
        return rng.uniform(-0.5, 0.5, size=shape)
    if dist == "normal1":
        return rng.standard_normal(size=shape)
    raise ValueError(dist)


def make_inputs(w: Workload, M: int | None = None, N: int | None = None, K: int | None = None,
                seed: int | None = None, layout_a: str | None = None,
                layout_b: str | None = None) -> dict:
    """Seeded inputs of workload ``w`` (optionally resized or re-laid-out).

    Returns dict with logical bit arrays ``a_bits`` (M x K) and ``b_bits`` (K x N), the
    stored flat arrays ``A`` and ``B`` in the requested layouts, and for int4 workloads
    ``B`` = packed codes and ``scales`` = binary16 bits [K/128][N].
    """
    M = w.M if M is None else M
    N = w.N if N is None else N
    K = w.K if K is None else K
    la = w.layout_a if layout_a is None else layout_a
    lb = w.layout_b if layout_b is None else layout_b
    rng = np.random.default_rng(1234 + w.index if seed is None else seed)
    out = {"M": M, "N": N, "K": K, "layout_a": la, "layout_b": lb}
    if w.int4:
        a = to_bits(rng.standard_normal(size=(M, K)), "f16")
        q = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
        s = to_bits(rng.uniform(0.005, 0.02, size=(K // 128, N)), "f16")
        out.update(a_bits=a, A=store(a, la), q=q, B=pack_u4_along_k(q), scales=s.reshape(-1),
                   layout_b="col")
        return out
    a = to_bits(_draw(rng, w.dist, (M, K), K), w.dtype_ab)
    b = to_bits(_draw(rng, w.dist, (K, N), K), w.dtype_ab)
    out.update(a_bits=a, b_bits=b, A=store(a, la), B=store(b, lb))
    return out


def integer_matrix(rng: np.random.Generator, rows: int, cols: int, lo: int, hi: int,
                   dtype: str) -> np.ndarray:
    """Integer-valued matrix with entries uniform in [lo, hi] as storage bits (exact in
    fp16/bf16 for |v| <= 256)."""
    return to_bits(rng.integers(lo, hi + 1, size=(rows, cols)).astype(np.float64), dtype)
