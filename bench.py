"""Benchmark of the operand-layout GEMM on one MI355X.

A step is one C = A*B of the 4096^3 fp16 GEMM in BLAS "NN" storage (A column-major, i.e.
M-contiguous and transposed in registers by the loader; B column-major, K-contiguous),
fp32 accumulate, fp16 output, inputs N(0,1)/sqrt(K), resident in HBM before timing.
Before the W warm-up steps, RAMP_MS of untimed launches bring the clock up from idle.

Prints one JSON line: the headline TFLOP/s, a roofline object for the GEMM kernel
(algorithmic 2*M*N*K flops per launch over the average launch duration measured with
HIP events on the launch stream), the CPU oracle's throughput on a bounded sample of
the same product, and the other workloads (other layouts, the non-power-of-2 bf16
GEMM, skinny split-K and int4 shapes in GB/s, the fp8 E4M3 4096^3 GEMM against the fp8
matrix peak, and the attention forward whose P*V takes V through the transposing loader)
under "workloads".

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--only-headline]
       python bench.py --copy-probe   (plain device copy of known size, for scaling
                                       rocprofv3 FETCH_SIZE / WRITE_SIZE counters)
       python bench.py --vendor-pair [--layout-a row|col --layout-b row|col] [--steps K]
                      (the 4096^3 fp16 GEMM, K calls of torch.mm (hipBLASLt) then K of this
                       library on the same operand bytes: for side-by-side rocprofv3 counters)
       python bench.py --workload NAME [--layout-a row|col --layout-b row|col] [--steps K]
                      (only that workload, K launches: the target of per-workload profiles;
                       for the attention workload --layout-a gives the dtype, f16 or bf16)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = 2500.0      # MI355X dense fp16/bf16 matrix peak
PEAK_F8_TFLOPS = 5000.0   # MI355X dense fp8 matrix peak
PEAK_GBS = 8000.0         # MI355X HBM3E
MALL_BYTES = 256 << 20    # Infinity Cache: HBM-bound timings rotate over more than 2x this
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_square_4096_nn.txt")
KERNEL_DIR = os.path.join(ROOT, "dense_gemm_operand_amd", "csrc")


# After an idle spell the GPU clock takes about 25 ms of back-to-back GEMM launches to reach
# its steady (power-limited) level: measured 4096^3 NN batches of 20 launches after a 1 s
# pause went 120, 138, 131, 121, ... 112 us and stayed at 111-112 us over 2000 launches.
# Every timing here first runs this long, untimed.
RAMP_MS = 60.0


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def ramp_up(fns, ms: float = RAMP_MS) -> None:
    """Launch the callables in turn, 10 calls each, untimed, until `ms` of wall time have
    passed with the GPU busy (synchronised after every turn), then synchronise."""
    import torch
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for fn in fns:
            for _ in range(10):
                fn()
        torch.cuda.synchronize()


def kernel_sha(folder: str = KERNEL_DIR) -> str:
    """Hash of the device-code sources (every .hpp and .hip under csrc, in name order) with
    comments and blank lines removed: counters taken on a build stay valid across comment
    edits, and become stale when any code line of any kernel changes."""
    code = []
    for name in sorted(os.listdir(folder)):
        if not name.endswith((".hpp", ".hip")):
            continue
        code.append("== " + name)
        with open(os.path.join(folder, name), encoding="utf-8") as f:
            for ln in f:
                ln = ln.split("//", 1)[0].rstrip()
                if ln:
                    code.append(ln)
    return hashlib.sha256("\n".join(code).encode()).hexdigest()[:16]


def read_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None when the
    summary is missing or was taken on a different kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for ln in open(TRAFFIC_FILE):
        if ":" in ln and not ln.startswith("#"):
            k, v = ln.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != kernel_sha():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class Gemm:
    """One planned GEMM with device operands (and rotation copies for HBM-bound shapes)."""

    def __init__(self, w, layout_a=None, layout_b=None, rotate_bytes=0, b_tiled=False):
        import torch
        import dense_gemm_operand_amd as dg
        from dense_gemm_operand_amd import synth
        self.dg, self.torch, self.w = dg, torch, w
        t0 = time.time()
        inp = synth.make_inputs(w, layout_a=layout_a, layout_b=layout_b)
        if b_tiled:   # int4 codes repacked into the pre-tiled layout (offline step)
            inp = dict(inp, B=dg.gemm_pack_u4_tiled(inp["B"], inp["N"], inp["K"]),
                       layout_b="u4_tiled")
        self.inp = inp
        self.M, self.N, self.K = inp["M"], inp["N"], inp["K"]
        self.la, self.lb = inp["layout_a"], inp["layout_b"]
        dev = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(
            np.int16 if x.dtype == np.uint16 else np.uint8)).cuda()
        A, B = dev(inp["A"]), dev(inp["B"])
        S = dev(inp["scales"]) if w.int4 else None
        self.in_bytes = A.numel() * A.element_size() + B.numel() * B.element_size() + \
            (S.numel() * S.element_size() if S is not None else 0)
        reps = 1
        if rotate_bytes:
            reps = max(1, -(-rotate_bytes // self.in_bytes))
        self.sets = [(A, B, S)] + [(A.clone(), B.clone(), S.clone() if S is not None else None)
                                   for _ in range(reps - 1)]
        self.plan = dg.gemm_plan(self.M, self.N, self.K, self.la, self.lb, w.dtype_ab,
                                 "u4" if w.int4 else w.dtype_ab, w.dtype_c, w.split_k,
                                 dg.int4_quant() if w.int4 else None)
        self.info = dg.gemm_plan_query(self.plan)
        ob = 4 if w.dtype_c == "f32" else 2
        self.C = torch.empty(self.M * self.N * ob // 2, dtype=torch.int16, device="cuda")
        nws = dg.gemm_workspace_size(self.plan)
        self.ws = torch.zeros(max(nws, 16), dtype=torch.uint8, device="cuda") if nws else None
        self.flops = 2.0 * self.M * self.N * self.K
        self.bytes = self.in_bytes + self.M * self.N * ob   # algorithmic: each operand once
        self.i = 0
        log(f"{w.name} {self.la}/{self.lb}: inputs ready in {time.time() - t0:.1f}s, "
            f"{len(self.sets)} set(s), plan tile={self.info['tile_m']}x{self.info['tile_n']} "
            f"split_k={self.info['split_k']}")

    def run(self):
        A, B, S = self.sets[self.i % len(self.sets)]
        self.i += 1
        self.dg.gemm_run(self.plan, A, B, S, self.C, self.ws)

    def time_b2b(self, n: int, warm_ms: float = RAMP_MS) -> float:
        """Average launch duration in ms: `n` back-to-back launches on the launch stream
        bracketed by one HIP event pair (the same way the headline's timed region is taken),
        after `warm_ms` of launches that bring the clock up from idle. Kernels shorter than
        50 us are timed with time_graph instead, so that the host's enqueue rate cannot enter
        the figure."""
        torch = self.torch
        ramp_up([self.run], warm_ms)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            self.run()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / n
        if ms < 0.05 and hasattr(self, "time_graph"):
            ms = self.time_graph()
        return ms

    def time_graph(self, launches: int = 32, replays: int = 10):
        """Average launch duration in ms for kernels too short for per-launch events: a
        HIP graph of `launches` back-to-back launches (rotating input sets) is captured on
        the launch stream and replayed; events bracket the replays. No host enqueue gap
        enters the figure."""
        torch = self.torch
        for _ in range(3):
            self.run()
        torch.cuda.synchronize()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            with torch.cuda.graph(graph, stream=s):
                for _ in range(launches):
                    self.run()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(replays):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (launches * replays)

    def close(self):
        self.dg.gemm_plan_destroy(self.plan)


class Attn:
    """One attention forward workload with device Q, K, V, O."""

    def __init__(self, w, dtype=None):
        import torch
        import dense_gemm_operand_amd as dg
        from dense_gemm_operand_amd import synth
        self.dg, self.torch, self.w = dg, torch, w
        inp = synth.make_attn_inputs(w, dtype=dtype)
        self.inp = inp
        dev = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda()
        self.Q, self.K, self.V = dev(inp["Q"]), dev(inp["K"]), dev(inp["V"])
        self.O = torch.empty_like(self.Q)
        self.args = (self.Q, self.K, self.V, self.O, inp["BH"], inp["Sq"], inp["Sk"], inp["D"],
                     inp["dtype"], inp["scale"])
        self.flops = 4.0 * inp["BH"] * inp["Sq"] * inp["Sk"] * inp["D"]

    def run(self):
        self.dg.attn_fwd(*self.args)

    time_b2b = Gemm.time_b2b


def cpu_baseline(g: Gemm, budget_s: float = 12.0):
    """The CPU leg: the oracle (untuned, all host threads) timed on a bounded sample, whole
    rows of the same product; the same rows then serve as a parity spot check of the GPU
    result. Returns (baseline, spot check)."""
    import oracle
    inp, w = g.inp, g.w
    t0 = time.time()
    a = oracle.operand_a(inp["A"], g.M, g.K, g.la, w.dtype_ab)
    b = oracle.operand_b(inp["B"], g.K, g.N, g.lb, "u4" if w.int4 else w.dtype_ab,
                         inp.get("scales"))
    prep = time.time() - t0
    probe = min(g.M, 2 * oracle.threads())
    t1 = time.time()
    oracle.gemm_f64(a, b, (0, probe))
    per_row = max((time.time() - t1) / probe, 1e-6)
    rows = int(max(1, min(g.M, (budget_s - prep) / per_row)))
    rng = np.random.default_rng(7)
    r0 = int(rng.integers(0, g.M - rows + 1))
    t2 = time.time()
    c64 = oracle.gemm_f64(a, b, (r0, r0 + rows))
    dt = time.time() - t2 + prep
    flops = 2.0 * rows * g.N * g.K
    baseline = {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.threads(),
                "kind": "oracle",
                "sample": f"rows {r0}..{r0 + rows - 1} of the {g.M}x{g.N}x{g.K} product "
                          f"({flops / 1e9:.1f} GFLOP, fp64, operand decode included, {dt:.1f}s)"}
    # parity spot check on the sampled rows
    g.run()
    g.torch.cuda.synchronize()
    fmt = g.w.dtype_c
    ob = 4 if fmt == "f32" else 2
    raw = g.C.cpu().numpy().view(np.uint32 if ob == 4 else np.uint16).reshape(g.M, g.N)
    got = oracle.decode(raw[r0:r0 + rows], fmt)
    ref = oracle.decode(oracle.encode(c64, fmt), fmt)
    rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    return baseline, {"rows": rows, "rel_frobenius": rel, "ok": rel <= 1e-3}


def stream_context() -> dict:
    """Device bandwidth context on the same box: a read-only pass (sum of a 2 GiB fp16
    tensor, far beyond the 256 MiB Infinity Cache) and a 1 GiB device copy (read + write)."""
    import torch
    x = torch.ones(1 << 30, dtype=torch.float16, device="cuda")
    y = torch.empty(1 << 29, dtype=torch.float16, device="cuda")
    z = torch.empty_like(y)
    for _ in range(2):
        x.sum()
        z.copy_(y)
    torch.cuda.synchronize()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    e[0].record()
    for _ in range(5):
        x.sum()
    e[1].record()
    for _ in range(5):
        z.copy_(y)
    e[2].record()
    torch.cuda.synchronize()
    rd = x.numel() * 2 * 5 / (e[0].elapsed_time(e[1]) * 1e-3) / 1e9
    cp = 2 * y.numel() * 2 * 5 / (e[1].elapsed_time(e[2]) * 1e-3) / 1e9
    del x, y, z
    torch.cuda.empty_cache()
    return {"stream_read_gbs": round(rd, 1), "copy_read_plus_write_gbs": round(cp, 1),
            "note": "torch sum over 2 GiB fp16 and copy of 1 GiB, events over 5 runs each"}


def interleaved(fns, rounds: int = 5, calls: int = 20) -> list:
    """Median ms per call of each callable, timed interleaved: rounds of `calls`
    back-to-back calls per callable, alternating, one event pair per batch, so that the
    power-limited clock affects every callable alike (after a ramp-up of all of them)."""
    import torch
    ramp_up(fns)
    t = [[] for _ in fns]
    for _ in range(rounds):
        for i, fn in enumerate(fns):
            for _ in range(3):
                fn()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(calls):
                fn()
            e1.record()
            torch.cuda.synchronize()
            t[i].append(e0.elapsed_time(e1) / calls)
    return [float(np.median(x)) for x in t]


def loader_comparison(rounds: int = 5, calls: int = 20) -> list:
    """The two loaders for transposed operands on the same shapes, timed interleaved: the
    in-register transpose (the default for NN; planner hooks DGEMM_FORCE_DTL=1
    DGEMM_FORCE_MFMA=16 for TT, DGEMM_FORCE_DTL=0 for NT) and direct-to-LDS loads in global
    order transposed by the LDS reads (the default for TT and NT; DGEMM_FORCE_DTL=2
    DGEMM_FORCE_MFMA=16 for NN). The default kernel's own time is the one under "workloads";
    here only the alternative's time and the ratio appear."""
    import torch
    from dense_gemm_operand_amd import synth
    res = []
    for name, la, lb in [("square_4096", "col", "col"), ("square_4096", "row", "row"),
                         ("square_4096", "col", "row"), ("nonpow2_bf16", None, None)]:
        wl = synth.WORKLOADS[name]
        pair = (la or wl.layout_a, lb or wl.layout_b)
        hs = []
        alt_env = {("col", "col"): {"DGEMM_FORCE_DTL": "2", "DGEMM_FORCE_MFMA": "16"},
                   ("row", "row"): {"DGEMM_FORCE_DTL": "1", "DGEMM_FORCE_MFMA": "16"},
                   ("col", "row"): {"DGEMM_FORCE_DTL": "0"}}[pair]
        for envs in ({}, alt_env):   # default first, then the other loader
            os.environ.update(envs)
            try:
                hs.append(Gemm(wl, la, lb))
            finally:
                for k in envs:
                    os.environ.pop(k, None)
        d, alt = interleaved([hs[0].run, hs[1].run], rounds, calls)
        loader = lambda h: "transposing_lds_reads" if h.info["direct_lds"] & 12 else "in_register_transpose"
        kern = lambda h: f"{h.info['tile_m']}x{h.info['tile_n']}, {h.info['mfma_m']}x{h.info['mfma_m']} blocks"
        rec = {"workload": name, "layout_a": hs[0].la, "layout_b": hs[0].lb,
               "default": loader(hs[0]), "alternative": loader(hs[1]),
               "default_kernel": kern(hs[0]), "alternative_kernel": kern(hs[1]),
               "alternative_us": round(alt * 1e3, 2),
               "alternative_over_default": round(alt / d, 4)}
        log(json.dumps(rec))
        res.append(rec)
        for h in hs:
            h.close()
        del hs
        torch.cuda.empty_cache()
    return res


def tile_comparison(rounds: int = 5, calls: int = 20) -> list:
    """The 3072x5120x6144 bf16 shape on its default plan (the non-power-of-2 192x320 tile:
    256 tiles, 8-wave ping-pong with 16x16x32 blocks, every operand straight into LDS)
    against 240 tiles of 256x256 on the 8-wave ping-pong with 32x32x16 blocks (planner hook
    DGEMM_FORCE_TILE=256x256), timed interleaved. The default's own time is the one under
    "workloads"; here only the alternative's time and the ratio appear."""
    import torch
    from dense_gemm_operand_amd import synth
    wl = synth.WORKLOADS["nonpow2_bf16"]
    hs = []
    for tile in (None, "256x256"):
        if tile is not None:
            os.environ["DGEMM_FORCE_TILE"] = tile
        try:
            hs.append(Gemm(wl))
        finally:
            os.environ.pop("DGEMM_FORCE_TILE", None)
    d, alt = interleaved([hs[0].run, hs[1].run], rounds, calls)
    desc = lambda h: (f"{h.info['tile_m']}x{h.info['tile_n']}, {h.info['waves']} waves, "
                      f"schedule {h.info['schedule']}, {h.info['mfma_m']}x{h.info['mfma_m']} "
                      f"blocks, direct_lds {h.info['direct_lds']}, grid {h.info['grid_x']}")
    rec = {"workload": wl.name, "layout_a": hs[0].la, "layout_b": hs[0].lb,
           "default": desc(hs[0]), "alternative": desc(hs[1]),
           "alternative_us": round(alt * 1e3, 2),
           "alternative_over_default": round(alt / d, 4)}
    log(json.dumps(rec))
    for h in hs:
        h.close()
    del hs
    torch.cuda.empty_cache()
    return [rec]


def _vendor_mm(h: "Gemm"):
    """torch.mm (hipBLASLt on ROCm) on the operand bytes of a planned fp16 GEMM, as a callable.
    The library's layouts as torch views of the same bytes: "row" A is [M][K], "col" A is
    [K][M]; "col" B is [N][K], "row" B is [K][N]."""
    import torch
    A, B, _ = h.sets[0]
    M, N, K = h.M, h.N, h.K
    ta = A.view(torch.float16).view(M, K) if h.la == "row" else A.view(torch.float16).view(K, M).t()
    tb = B.view(torch.float16).view(N, K).t() if h.lb == "col" else B.view(torch.float16).view(K, N)
    out = torch.empty(M, N, dtype=torch.float16, device="cuda")
    return lambda: torch.mm(ta, tb, out=out)


def vendor_blas_comparison(rounds: int = 5, calls: int = 20) -> list:
    """Context, not a result: torch.mm (which dispatches to the vendor hipBLASLt kernels on
    ROCm) on the same operand memory as the 4096^3 fp16 GEMM in each layout, and
    torch._scaled_mm against the fp8 E4M3 one in the layout it takes (TN), timed
    interleaved with this library. This library's own times are under "workloads"; here
    the vendor's time and the ratio vendor / this library."""
    import torch
    from dense_gemm_operand_amd import synth
    wl = synth.WORKLOADS["square_4096"]
    res = []
    for la, lb in [("col", "col"), ("row", "col"), ("row", "row"), ("col", "row")]:
        h = Gemm(wl, la, lb)
        ours, blas = interleaved([h.run, _vendor_mm(h)], rounds, calls)
        rec = {"workload": wl.name, "layout_a": la, "layout_b": lb,
               "torch_mm_us": round(blas * 1e3, 2), "torch_mm_over_this": round(blas / ours, 4)}
        log(json.dumps(rec))
        res.append(rec)
        h.close()
        del h
        torch.cuda.empty_cache()
    wl8 = synth.WORKLOADS["square_4096_f8"]
    h = Gemm(wl8, "row", "col")
    A, B, _ = h.sets[0]
    f8 = torch.float8_e4m3fn
    ta = A.view(f8).view(h.M, h.K)
    tb = B.view(f8).view(h.N, h.K).t()
    one = torch.tensor(1.0, device="cuda")
    ours, blas = interleaved([h.run, lambda: torch._scaled_mm(ta, tb, scale_a=one, scale_b=one,
                                                              out_dtype=torch.float16)],
                             rounds, calls)
    rec = {"workload": wl8.name, "layout_a": "row", "layout_b": "col",
           "torch_scaled_mm_us": round(blas * 1e3, 2), "torch_scaled_mm_over_this": round(blas / ours, 4)}
    log(json.dumps(rec))
    res.append(rec)
    h.close()
    del h, ta, tb
    torch.cuda.empty_cache()
    return res


def int4_layout_comparison(rounds: int = 5) -> list:
    """int4 B pre-tiled (64 columns x 128 K blocks) against the column-major packing (the
    workload's own layout, timed under "workloads"), interleaved: HIP graphs of
    back-to-back launches over rotating input sets for M = 16, back-to-back launches for
    M = 4096. Reports the pre-tiled time and the ratio."""
    import torch
    from dense_gemm_operand_amd import synth
    res = []
    for name in ("int4_m16", "int4_m4096"):
        wl = synth.WORKLOADS[name]
        hbm = name == "int4_m16"
        rot = 2 * MALL_BYTES + (64 << 20) if hbm else 0
        hs = [Gemm(wl, rotate_bytes=rot), Gemm(wl, rotate_bytes=rot, b_tiled=True)]
        if hbm:
            t = [[], []]
            ramp_up([h.run for h in hs])
            for _ in range(rounds):
                for i, h in enumerate(hs):
                    t[i].append(h.time_graph(32, 5))
            col, tiled = float(np.median(t[0])), float(np.median(t[1]))
        else:
            col, tiled = interleaved([hs[0].run, hs[1].run], rounds, 10)
        h = hs[1]
        rec = {"workload": name, "M": h.M, "N": h.N, "K": h.K,
               "pre_tiled_us": round(tiled * 1e3, 2),
               "pre_tiled_gbs": round(h.bytes / (tiled * 1e-3) / 1e9, 1),
               "pre_tiled_tflops": round(h.flops / (tiled * 1e-3) / 1e12, 1),
               "pre_tiled_over_column_major": round(tiled / col, 4),
               "split_k": h.info["split_k"], "tile": f"{h.info['tile_m']}x{h.info['tile_n']}"}
        log(json.dumps(rec))
        res.append(rec)
        for h in hs:
            h.close()
        del hs
        torch.cuda.empty_cache()
    return res


def cpu_baselines(budget_s: float = 2.5) -> list:
    """The oracle (untuned, all host threads) on a bounded sample of every workload and
    layout: whole output rows, sized so that each takes about `budget_s` seconds including
    the decode (and int4 dequant) of the operands. A reported baseline, not a target."""
    import oracle
    from dense_gemm_operand_amd import synth
    res = []
    cases = [("square_tt_256", None, None)] + \
        [("square_4096", la, lb) for la, lb in synth.LAYOUT_LETTERS.values()] + \
        [("nonpow2_bf16", None, None), ("skinny_splitk", None, None), ("int4_m16", None, None),
         ("int4_m4096", None, None), ("square_4096_f8", None, None)]
    for name, la, lb in cases:
        w = synth.WORKLOADS[name]
        inp = synth.make_inputs(w, layout_a=la, layout_b=lb)
        M, N, K = inp["M"], inp["N"], inp["K"]
        t0 = time.time()
        a = oracle.operand_a(inp["A"], M, K, inp["layout_a"], w.dtype_ab)
        b = oracle.operand_b(inp["B"], K, N, inp["layout_b"], "u4" if w.int4 else w.dtype_ab,
                             inp.get("scales"))
        prep = time.time() - t0
        probe = min(M, max(1, oracle.threads()))
        t1 = time.time()
        oracle.gemm_f64(a, b, (0, probe))
        per_row = max((time.time() - t1) / probe, 1e-7)
        rows = int(max(1, min(M, (budget_s - prep) / per_row)))
        t2 = time.time()
        oracle.gemm_f64(a, b, (0, rows))
        dt = time.time() - t2 + prep
        flops = 2.0 * rows * N * K
        rec = {"workload": name, "layout_a": inp["layout_a"], "layout_b": inp["layout_b"],
               "M": M, "N": N, "K": K, "rows": rows, "seconds": round(dt, 3),
               "gmacs": round(flops / 2 / dt / 1e9, 3), "tflops": round(flops / dt / 1e12, 6),
               "cores": oracle.threads(), "kind": "oracle"}
        log(json.dumps(rec))
        res.append(rec)
        del a, b, inp
    return res


def run_workload(name: str, la, lb, steps: int):
    """Only one workload: RAMP_MS of untimed launches, then `steps` launches (rotating input
    sets for HBM-bound shapes). A profile of it averages the last `steps` dispatches."""
    import torch
    from dense_gemm_operand_amd import synth
    if name in synth.ATTN_WORKLOADS:
        aw = synth.ATTN_WORKLOADS[name]
        at = Attn(aw, la)   # --layout-a doubles as the attention dtype (f16 / bf16)
        ramp_up([at.run])
        for _ in range(steps):
            at.run()
        torch.cuda.synchronize()
        print(json.dumps({"workload": name, "dtype": at.inp["dtype"], "launches": steps,
                          "batch_heads": aw.BH, "seq_q": aw.seq_q, "seq_k": aw.seq_k,
                          "head_dim": aw.head_dim}), flush=True)
        return
    wl = synth.WORKLOADS[name]
    hbm = name in ("skinny_splitk", "int4_m16")
    g = Gemm(wl, la, lb, rotate_bytes=2 * MALL_BYTES + (64 << 20) if hbm else 0)
    ramp_up([g.run])
    for _ in range(steps):
        g.run()
    torch.cuda.synchronize()
    print(json.dumps({"workload": name, "layout_a": g.la, "layout_b": g.lb, "launches": steps,
                      "tile": f"{g.info['tile_m']}x{g.info['tile_n']}", "waves": g.info["waves"],
                      "split_k": g.info["split_k"], "direct_lds": g.info["direct_lds"],
                      "perm_block": g.info["perm_block"]}), flush=True)
    g.close()


def copy_probe():
    import torch
    n = 256 << 20
    src = torch.ones(n // 2, dtype=torch.int16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n}))


def vendor_pair(la: str | None, lb: str | None, calls: int):
    """`calls` launches of the vendor library's product, then `calls` of this library's, on
    the same operand memory of the 4096^3 fp16 GEMM (one layout pair, default TN), each after
    RAMP_MS of untimed launches of its own."""
    import torch
    from dense_gemm_operand_amd import synth
    h = Gemm(synth.WORKLOADS["square_4096"], la or "row", lb or "col")
    mm = _vendor_mm(h)
    ramp_up([mm])
    for _ in range(calls):
        mm()
    torch.cuda.synchronize()
    ramp_up([h.run])
    for _ in range(calls):
        h.run()
    torch.cuda.synchronize()
    print(json.dumps({"vendor_pair": f"{h.la}/{h.lb}", "calls": calls}))
    h.close()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # (the headline runs RAMP_MS of untimed launches before its W warm-up steps)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--only-headline", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--vendor-pair", action="store_true")
    ap.add_argument("--workload", default=None)
    ap.add_argument("--layout-a", default=None)
    ap.add_argument("--layout-b", default=None)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library runs on a single MI355X and has no "
              f"multi-GPU path (asked for --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_probe:
        copy_probe()
        return
    if args.vendor_pair:
        vendor_pair(args.layout_a, args.layout_b, args.steps)
        return
    if args.workload:
        run_workload(args.workload, args.layout_a, args.layout_b, args.steps)
        return
    from dense_gemm_operand_amd import synth
    torch.cuda.set_device(0)

    w = synth.WORKLOADS["square_4096"]
    g = Gemm(w, "col", "col")
    # The clock's ramp from idle first (RAMP_MS of untimed launches, whatever --warmup says:
    # a short warm-up would otherwise leave the timed region inside the ramp), then the W
    # warm-up steps.
    ramp_up([g.run])
    for _ in range(args.warmup):
        g.run()
    torch.cuda.synchronize()
    # The timed region: K back-to-back launches on the launch stream (torch's current
    # stream), bracketed by a host clock and by one HIP event pair on that stream.
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        g.run()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    value = g.flops / (ms_step * 1e-3) / 1e12
    kern_ms = e0.elapsed_time(e1) / args.steps
    achieved = g.flops / (kern_ms * 1e-3) / 1e12
    log(f"headline: wall {ms_step * 1e3:.1f} us/step, events over the same region "
        f"{kern_ms * 1e3:.1f} us/launch -> {achieved:.1f} TFLOP/s")

    out = {
        "metric": "TFLOP/s and % of dense MFMA peak, 4096^3 NN fp16 GEMM; GB/s for split-K",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_ramp_ms": RAMP_MS,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "fp16 GEMM 4096x4096x4096, BLAS NN (A M-contiguous, B "
                               "K-contiguous), fp32 accumulate, fp16 out, N(0,1)/sqrt(K)",
                   "M": 4096, "N": 4096, "K": 4096, "layout_a": "col", "layout_b": "col",
                   "tile": f"{g.info['tile_m']}x{g.info['tile_n']}x{g.info['tile_k']}",
                   "waves": g.info["waves"], "split_k": g.info["split_k"]},
        "pct_of_peak": round(100.0 * value / PEAK_TFLOPS, 2),
    }
    traffic = read_traffic()
    out["roofline"] = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_TFLOPS,
                       "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS, 4),
                       "traffic": traffic,
                       "kernel_avg_us": round(kern_ms * 1e3, 2),
                       "flops_per_launch": g.flops,
                       "timing": "HIP events on the launch stream around the timed region, "
                                 "divided by the launches in it"}
    if not args.no_cpu:
        out["cpu_baseline"], out["parity_spot_check"] = cpu_baseline(g)
    g.close()
    del g
    torch.cuda.empty_cache()

    if not args.only_headline:
        extra = []
        # (workload, layouts, bound); the headline NN layout is timed above
        cases = [
            ("square_4096", "row", "row", "mfma"), ("square_4096", "col", "row", "mfma"),
            ("square_4096", "row", "col", "mfma"), ("nonpow2_bf16", None, None, "mfma"),
            ("square_tt_256", None, None, "mfma"), ("int4_m4096", None, None, "mfma"),
            ("skinny_splitk", None, None, "hbm"), ("int4_m16", None, None, "hbm"),
            ("square_4096_f8", None, None, "mfma"), ("square_4096_f8", "row", "col", "mfma"),
        ]
        for name, la, lb, bound in cases:
            wl = synth.WORKLOADS[name]
            rot = 2 * MALL_BYTES + (64 << 20) if bound == "hbm" else 0
            h = Gemm(wl, la, lb, rotate_bytes=rot)
            ms = h.time_b2b(100 if bound == "hbm" else 50)
            rec = {"workload": name, "M": h.M, "N": h.N, "K": h.K, "layout_a": h.la,
                   "layout_b": h.lb, "dtype": wl.dtype_ab + ("+u4" if wl.int4 else ""),
                   "out": wl.dtype_c, "split_k": h.info["split_k"],
                   "tile": f"{h.info['tile_m']}x{h.info['tile_n']}", "kernel": h.info["kernel"],
                   "us": round(ms * 1e3, 2),
                   "tflops": round(h.flops / (ms * 1e-3) / 1e12, 2),
                   "gbs": round(h.bytes / (ms * 1e-3) / 1e9, 1),
                   "input_sets": len(h.sets),
                   "loader": ("transposing LDS reads" if h.info["direct_lds"] & 12 else
                              "in-register transpose" if (h.la == "col" or h.lb == "row") else
                              "K-contiguous"),
                   "direct_lds": h.info["direct_lds"], "waves": h.info["waves"],
                   "schedule": h.info["schedule"], "mfma_m": h.info["mfma_m"]}
            peak = PEAK_F8_TFLOPS if wl.dtype_ab == "f8" else PEAK_TFLOPS
            rec["pct_peak"] = round(100 * (rec["tflops"] / peak if bound == "mfma"
                                           else rec["gbs"] / PEAK_GBS), 2)
            rec["bound"] = bound
            log(json.dumps(rec))
            extra.append(rec)
            h.close()
            del h
            torch.cuda.empty_cache()
        for dt in ("f16", "bf16"):
            aw = synth.ATTN_WORKLOADS["attn_4096"]
            at = Attn(aw, dt)
            ms = at.time_b2b(30)
            rec = {"workload": aw.name, "batch_heads": aw.BH, "seq_q": aw.seq_q, "seq_k": aw.seq_k,
                   "head_dim": aw.head_dim, "dtype": dt, "us": round(ms * 1e3, 2),
                   "tflops": round(at.flops / (ms * 1e-3) / 1e12, 2),
                   "pct_peak": round(100 * at.flops / (ms * 1e-3) / 1e12 / PEAK_TFLOPS, 2),
                   "bound": "mfma", "loader": "V transposed in registers (attention P*V)"}
            log(json.dumps(rec))
            extra.append(rec)
            del at
            torch.cuda.empty_cache()
        out["workloads"] = extra
        out["timing"] = ("every time above: back-to-back launches bracketed by one HIP event "
                         "pair on the launch stream (HIP graph replays for kernels under 50 "
                         "us); the comparisons below give ratios from interleaved batches")
        out["loader_comparison"] = loader_comparison()
        out["tile_comparison"] = tile_comparison()
        out["int4_layout_comparison"] = int4_layout_comparison()
        out["vendor_blas_comparison"] = vendor_blas_comparison()
        out["context"] = stream_context()
        if not args.no_cpu:
            out["cpu_baseline_per_workload"] = cpu_baselines()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
