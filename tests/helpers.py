"""Shared test helpers: run the HIP path through the C ABI and compare with the oracle."""
from __future__ import annotations

import contextlib
import os

import numpy as np

import oracle

FMT_BYTES = {"f32": 4, "f16": 2, "bf16": 2}


@contextlib.contextmanager
def env(**kv):
    """Temporarily set planner hooks (DGEMM_FORCE_TILE etc.) in the environment."""
    old = {k: os.environ.get(k) for k in kv}
    try:
        for k, v in kv.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = str(v)
        yield
    finally:
        for k, v in old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


def to_dev(x: np.ndarray):
    import torch
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        t = torch.from_numpy(x.view(np.int16))
    elif x.dtype == np.uint8:
        t = torch.from_numpy(x)
    else:
        raise TypeError(x.dtype)
    return t.cuda()


def run_gpu(inp: dict, dtype_ab: str, dtype_c: str, split_k: int = 0, int4: bool = False,
            guard: int = 0, repeat: int = 1, force_tile: str | None = None,
            force_split_k: int | None = None, group: int = 128, zero: int = 8):
    """Plan + run C = A*B on the GPU through the C ABI; returns (C bits, plan info).

    ``guard`` extra sentinel elements are allocated after C and checked untouched."""
    import torch
    import dense_gemm_operand_amd as dg
    M, N, K = inp["M"], inp["N"], inp["K"]
    with env(DGEMM_FORCE_TILE=force_tile, DGEMM_FORCE_SPLIT_K=force_split_k):
        plan = dg.gemm_plan(M, N, K, inp["layout_a"], inp["layout_b"], dtype_ab,
                            "u4" if int4 else dtype_ab, dtype_c, split_k,
                            dg.int4_quant(group, zero) if int4 else None)
    try:
        info = dg.gemm_plan_query(plan)
        A = to_dev(inp["A"])
        B = to_dev(inp["B"])
        S = to_dev(inp["scales"]) if int4 else None
        eb = FMT_BYTES[dtype_c]
        cdt = torch.int32 if eb == 4 else torch.int16
        sentinel = 0x5A5A5A5A if eb == 4 else 0x5A5A
        Cfull = torch.full((M * N + guard,), sentinel, dtype=cdt, device="cuda")
        ws_bytes = dg.gemm_workspace_size(plan)
        ws = torch.zeros(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
        outs = []
        for _ in range(repeat):
            dg.gemm_run(plan, A, B, S, Cfull, ws if ws_bytes else None)
            torch.cuda.synchronize()
            outs.append(Cfull[: M * N].cpu().numpy().copy())
        if guard:
            tail = Cfull[M * N:].cpu().numpy()
            assert np.all(tail == np.array(sentinel).astype(tail.dtype)), "write past the end of C"
        if ws_bytes:
            cnt = ws[: dg.COUNTER_BYTES].cpu().numpy()
            assert not cnt.any(), "split-K counters not reset"
        view = np.uint32 if eb == 4 else np.uint16
        outs = [o.view(view).reshape(M, N) for o in outs]
        return (outs if repeat > 1 else outs[0]), info
    finally:
        dg.gemm_plan_destroy(plan)


def reference(inp: dict, dtype_ab: str, dtype_c: str, int4: bool = False, rows=None,
              group: int = 128, zero: int = 8):
    """Oracle C (fp64 sums, and bits rounded to dtype_c) for the given inputs."""
    M, N, K = inp["M"], inp["N"], inp["K"]
    return oracle.gemm(inp["A"], inp["B"], M, N, K, inp["layout_a"], inp["layout_b"], dtype_ab,
                       dtype_c, scales_bits=inp.get("scales") if int4 else None, rows=rows,
                       group=group, zero=zero)


def operand_max(inp: dict, dtype_ab: str, int4: bool = False):
    a = oracle.decode(inp["A"], dtype_ab)
    if int4:
        b = oracle.dequant_u4(inp["B"], inp["scales"], inp["K"], inp["N"])
    else:
        b = oracle.decode(inp["B"], dtype_ab)
    return float(np.abs(a).max()), float(np.abs(b).max())


def check_tolerance(c_gpu_bits, c_ref_bits, dtype_c: str, K: int, amax: float, bmax: float,
                    what: str = ""):
    """The acceptance bar: relative Frobenius error <= 1e-3 against the oracle rounded to the
    output format, and every element within 4e-3 * sqrt(K) * max|a| * max|b|."""
    g = oracle.decode(np.ascontiguousarray(c_gpu_bits), dtype_c)
    r = oracle.decode(np.ascontiguousarray(c_ref_bits), dtype_c)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    denom = np.linalg.norm(r)
    rel = np.linalg.norm(g - r) / denom if denom > 0 else np.linalg.norm(g)
    bound = 4e-3 * np.sqrt(K) * amax * bmax
    worst = float(np.abs(g - r).max()) if g.size else 0.0
    assert rel <= 1e-3, f"{what}: relative Frobenius error {rel:.3e}"
    assert worst <= bound, f"{what}: max element error {worst:.3e} > {bound:.3e}"
    return rel, worst
