"""Benchmark: FP4 quantized linear layer forward on one MI355X.

One step = one fp4lin_forward call: the whole forward over one batch (outlier
select giving tau and the COO of dA, token-wise quantization of A, channel-wise
quantization of W, the FP4 GEMM with its scale epilogue, and the sparse
compensation Y += dA.W). The timed region is exactly K such calls. A second
loop issues the same work as the separate public calls with HIP events between
them on the stream the kernels run on, for the per-stage breakdown and the
per-kernel rooflines.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--pass forward|dgrad|wgrad]
                    [--quant token|mx]

Prints one JSON line. Inputs are seeded synthetic matrices (workloads module),
already resident in HBM when the timed region starts.

--pass dgrad / wgrad time the backward GEMMs of the same layer instead, each
step being its three public calls: dX = Q(dY) Q(W)^T (quantize_act on dY and on
W rows, then gemm) or dW = Q(A)^T Q(dY) (quantize_weight on A and on dY, then
gemm with K' = M).

--quant mx times the micro-scaled variant of the forward instead: each step is
one fp4lin_forward_mx call (32-code blocks along K with E8M0 scales, the block
scales applied by the matrix core); the per-stage breakdown issues its five
public calls outlier_select, quantize_act_mx, quantize_weight_mx, gemm_mx and
sparse_add. With --pass dgrad / wgrad it takes the
micro-scaled quantizers and gemm_mx for the backward GEMMs (blocks along the
reduction: N for dgrad, M for wgrad).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FP4 linear fwd effective TFLOP/s + % FP4 MFMA peak (7B FFN shape, 1 GPU)"
FP4_PEAK_TFLOPS = 10100.0   # MI355X dense FP4 MFMA
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E
# fp32 FMA on the vector ALUs without packed math: 256 CUs x 4 SIMDs x 16 lanes
# x 2 flop x 2.4 GHz (the 157.3 TFLOP/s figure needs packed fp32 FMA, which this
# library does not use)
VALU_FP32_PEAK_TFLOPS = 78.6


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="llama7b_ffn_up")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-rows", type=int, default=0,
                   help="rows of A in the CPU-oracle sample (0 = the whole workload)")
    p.add_argument("--copy-calib", action="store_true",
                   help="also run a plain 1 GiB device copy (for PMC byte calibration)")
    p.add_argument("--pass", dest="which", default="forward",
                   choices=("forward", "dgrad", "wgrad"))
    p.add_argument("--quant", default="token", choices=("token", "mx"),
                   help="token: the vector-wise forward (default); mx: the micro-scaled one")
    p.add_argument("--no-13b", action="store_true",
                   help="skip the 13B FFN up/down forwards the default run reports beside 7B")
    return p.parse_args()


# the GEMM runs the compensation in its epilogue up to this many COO entries
# per row of A (the COO capacity bounds them), else as a second kernel
FUSED_MAX_PER_ROW = 10


def forward_rate(L, dev, steps, warmup):
    """Back-to-back fp4lin_forward calls on layer L (inputs resident in HBM):
    ms per forward from HIP events on the stream the kernels run on."""
    import torch
    import quantized_linear_layer_amd as ql
    import workloads as wl
    A, W = upload(L.A, dev), upload(L.W, dev)
    stream = torch.cuda.current_stream()
    st = Step(ql, A, W, L.q, stream)
    for _ in range(max(warmup, 1)):
        st.forward_call()
    torch.cuda.synchronize()
    nnz = int(st.ws[st.offsets.row_ptr + 4 * L.M: st.offsets.row_ptr + 4 * L.M + 4]
              .cpu().numpy().view(np.int32)[0])
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        st.forward_call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    flops = 2.0 * L.M * L.N * L.K
    tf = flops / (ms * 1e-3) / 1e12
    fused = st.offsets.capacity <= FUSED_MAX_PER_ROW * L.M
    return {"M": L.M, "K": L.K, "N": L.N, "q": L.q, "nnz_dA": nnz, "ms": round(ms, 5),
            "TFLOP/s": round(tf, 1), "pct_fp4_peak": round(100.0 * tf / FP4_PEAK_TFLOPS, 2),
            "compensation": "gemm epilogue" if fused else "separate kernel", "steps": steps}


def file_sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


class Step:
    """Marshals the four stage calls once; each call is then a bare C call."""

    def __init__(self, ql, A, W, q, stream):
        import torch
        self.torch = torch
        self.ql = ql
        lib = ql.lib()
        self.lib = lib
        M, K = A.shape
        N = W.shape[1]
        dt = ql.BF16 if A.dtype == torch.bfloat16 else ql.F32
        self.M, self.K, self.N, self.q = M, K, N, q
        o = ql.forward_layout(M, K, N, dt, q)
        self.ws = torch.empty(o.total, dtype=torch.uint8, device=A.device)
        self.Y = torch.empty((M, N), dtype=torch.float32, device=A.device)
        base = self.ws.data_ptr()
        P = ctypes.c_void_p
        self.tau = P(base + o.tau)
        self.coo = ql.Coo(base + o.coo_row, base + o.coo_col, base + o.coo_val,
                          base + o.row_ptr, o.capacity)
        self.Aq, self.sA = P(base + o.Aq), P(base + o.sA)
        self.Wq, self.sW = P(base + o.Wq), P(base + o.sW)
        self.scratch, self.scratch_bytes = P(base + o.scratch), o.total - o.scratch
        self.A, self.W = P(A.data_ptr()), P(W.data_ptr())
        self.lda, self.ldw = A.stride(0), W.stride(0)
        self.dt = dt
        self.stream = P(stream.cuda_stream)
        self.offsets = o

    def select(self):
        s = self.lib.fp4lin_outlier_select(self.A, self.dt, self.M, self.K, self.lda, self.q,
                                           self.tau, self.coo, self.scratch, self.scratch_bytes,
                                           self.stream)
        assert s == 0, s

    def quant_a(self):
        s = self.lib.fp4lin_quantize_act(self.A, self.dt, self.M, self.K, self.lda, self.tau,
                                         self.Aq, self.sA, self.stream)
        assert s == 0, s

    def quant_w(self):
        s = self.lib.fp4lin_quantize_weight(self.W, self.dt, self.K, self.N, self.ldw, self.Wq,
                                            self.sW, self.scratch, self.scratch_bytes, self.stream)
        assert s == 0, s

    def gemm(self):
        s = self.lib.fp4lin_gemm(self.Aq, self.sA, self.Wq, self.sW, self.M, self.N, self.K,
                                 None, None, self.dt, 0, ctypes.c_void_p(self.Y.data_ptr()),
                                 self.N, self.stream)
        assert s == 0, s

    def sparse(self):
        s = self.lib.fp4lin_sparse_add(ctypes.byref(self.coo), self.W, self.dt, self.K, self.ldw,
                                       self.M, self.N, ctypes.c_void_p(self.Y.data_ptr()),
                                       self.N, self.stream)
        assert s == 0, s

    def forward_call(self):
        s = self.lib.fp4lin_forward(self.A, self.W, self.dt, self.M, self.K, self.N, self.lda,
                                    self.ldw, self.q, ctypes.c_void_p(self.Y.data_ptr()), self.N,
                                    ctypes.c_void_p(self.ws.data_ptr()), self.ws.numel(),
                                    self.stream)
        assert s == 0, s


class MxStep(Step):
    """The micro-scaled forward as its five public calls: the select's outputs
    and the packed codes live in the forward layout, the E8M0 scale rows in
    their own buffers."""

    def __init__(self, ql, A, W, q, stream):
        super().__init__(ql, A, W, q, stream)
        nb = ql.mx_scales_ld(self.K)   # scale bytes per row (stored step-major)
        self.As_t = self.torch.empty((self.M * nb,), dtype=self.torch.uint8, device=A.device)
        self.Ws_t = self.torch.empty((self.N * nb,), dtype=self.torch.uint8, device=A.device)
        self.As = ctypes.c_void_p(self.As_t.data_ptr())
        self.Ws = ctypes.c_void_p(self.Ws_t.data_ptr())
        # fp4lin_forward_mx's own workspace
        nbytes = int(self.lib.fp4lin_workspace_bytes_mx(self.M, self.K, self.N, self.dt, q))
        self.mws = self.torch.empty((nbytes,), dtype=self.torch.uint8, device=A.device)

    def quant_a(self):
        s = self.lib.fp4lin_quantize_act_mx(self.A, self.dt, self.M, self.K, self.lda, self.tau,
                                            self.Aq, self.As, self.stream)
        assert s == 0, s

    def quant_w(self):
        s = self.lib.fp4lin_quantize_weight_mx(self.W, self.dt, self.K, self.N, self.ldw,
                                               self.Wq, self.Ws, self.stream)
        assert s == 0, s

    def gemm(self):
        s = self.lib.fp4lin_gemm_mx(self.Aq, self.As, self.Wq, self.Ws, self.M, self.N, self.K,
                                    None, None, self.dt, 0, ctypes.c_void_p(self.Y.data_ptr()),
                                    self.N, self.stream)
        assert s == 0, s

    def step(self):
        s = self.lib.fp4lin_forward_mx(self.A, self.W, self.dt, self.M, self.K, self.N,
                                       self.lda, self.ldw, self.q,
                                       ctypes.c_void_p(self.Y.data_ptr()), self.N,
                                       ctypes.c_void_p(self.mws.data_ptr()), self.mws.numel(),
                                       self.stream)
        assert s == 0, s


def run_forward_mx(args):
    """One JSON line for --quant mx: the micro-scaled forward, step = one
    fp4lin_forward_mx call."""
    import torch
    import quantized_linear_layer_amd as ql
    import workloads as wl
    dev = torch.device("cuda:0")
    L = wl.make_layer(args.workload, seed=args.seed)
    A, W = upload(L.A, dev), upload(L.W, dev)
    stream = torch.cuda.current_stream()
    st = MxStep(ql, A, W, L.q, stream)
    M, K, N = L.M, L.K, L.N
    flops = 2.0 * M * N * K
    for _ in range(max(args.warmup, 1)):
        st.select(); st.quant_a(); st.quant_w(); st.gemm(); st.sparse()
        st.step()
    torch.cuda.synchronize()
    nnz = int(st.ws[st.offsets.row_ptr + 4 * M: st.offsets.row_ptr + 4 * M + 4]
              .cpu().numpy().view(np.int32)[0])
    f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    f0.record(stream)
    for _ in range(args.steps):
        st.step()
    f1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    event_ms = f0.elapsed_time(f1) / args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(STAGES) + 1)]
          for _ in range(args.steps)]
    for i in range(args.steps):
        e = ev[i]
        e[0].record(stream)
        st.select(); e[1].record(stream)
        st.quant_a(); e[2].record(stream)
        st.quant_w(); e[3].record(stream)
        st.gemm(); e[4].record(stream)
        st.sparse(); e[5].record(stream)
    torch.cuda.synchronize()
    stage_ms = {n: float(np.mean([ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(args.steps)]))
                for j, n in enumerate(STAGES)}
    if args.copy_calib:
        copy_calibration(dev)
    value = flops / (ms_per_step * 1e-3) / 1e12
    e = 2 if L.A.dtype == wl.BF16 else 4
    ldq = ql.packed_ld(K)
    nb = ql.mx_scales_ld(K)
    # algorithmic bytes: as the token-wise forward, with a scale row of nb
    # bytes per row of A and column of W instead of one float
    hbm_bytes = {
        "select": 2 * e * M * K + 12 * nnz + 4 * (M + 1),
        "quant_a": e * M * K + M * (ldq + nb),
        "quant_w": e * K * N + N * (ldq + nb),
        "gemm": (M + N) * (ldq + nb) + 4 * M * N,
        "sparse": 8 * M * N + 12 * nnz + 4 * (M + 1) + e * N * min(K, nnz),
    }
    kernels = {}
    for name in STAGES:
        gbs = hbm_bytes[name] / (stage_ms[name] * 1e-3) / 1e9
        kernels[name] = {"ms": round(stage_ms[name], 5), "bytes": int(hbm_bytes[name]),
                         "GB/s": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                         "bound": "hbm"}
    gemm_tf = flops / (stage_ms["gemm"] * 1e-3) / 1e12
    kernels["gemm"].update({"bound": "mfma", "TFLOP/s": round(gemm_tf, 1),
                            "mfma_frac": round(gemm_tf / FP4_PEAK_TFLOPS, 4)})
    sp_tf = 2.0 * nnz * N / (stage_ms["sparse"] * 1e-3) / 1e12
    kernels["sparse"].update({"bound": "alu", "fp32_TFLOP/s": round(sp_tf, 2),
                              "alu_frac": round(sp_tf / VALU_FP32_PEAK_TFLOPS, 4)})
    dom = max(STAGES, key=lambda n: stage_ms[n])
    traffic = None
    tname = {"gemm": f"traffic_gemm_{args.workload}_mx.json",
             "sparse": f"traffic_sparse_{args.workload}_mx.json"}.get(dom)
    if tname and os.path.exists(os.path.join(ROOT, "profiles", tname)):
        tr = json.load(open(os.path.join(ROOT, "profiles", tname)))
        if tr.get("source_sha256") == file_sha(os.path.join(ROOT, tr["source"])):
            traffic = tr.get("bytes_per_launch")
    if dom == "sparse":
        roof = {"bound": "alu", "kernel": "sparse_add_kernel", "achieved": round(sp_tf, 2),
                "peak": VALU_FP32_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(sp_tf / VALU_FP32_PEAK_TFLOPS, 4), "traffic": traffic}
    elif dom == "gemm":
        roof = {"bound": "mfma", "kernel": "fp4_gemm_kernel (block scales)",
                "achieved": round(gemm_tf, 2), "peak": FP4_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(gemm_tf / FP4_PEAK_TFLOPS, 4), "traffic": traffic}
    else:
        roof = {"bound": "hbm", "kernel": dom, "achieved": kernels[dom]["GB/s"],
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": kernels[dom]["hbm_frac"],
                "traffic": None}
    out = {
        "metric": "FP4 linear fwd effective TFLOP/s, micro-scaled operands (MXFP4, 32-code "
                  "E8M0 blocks; 1 GPU)",
        "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp4", "data": "synthetic",
        "config": {"workload": f"{args.workload}_mx", "M": M, "K": K, "N": N, "q": L.q,
                   "input_dtype": L.A.dtype, "output_dtype": "f32", "seed": args.seed,
                   "nnz_dA": nnz, "block": 32},
        "pct_fp4_peak": round(100.0 * value / FP4_PEAK_TFLOPS, 2),
        "event_ms": round(event_ms, 5),
        "stage_ms": {k: round(v, 5) for k, v in stage_ms.items()},
        "roofline": roof,
        "kernels": kernels,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_mx(L, args.cpu_rows or 256)
    print(json.dumps(out), flush=True)


def cpu_baseline_mx(L, rows):
    """The oracle's micro-scaled forward on the first `rows` rows of A (tau from
    those rows; W quantized whole), timed on the host cores."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()
                            if i.get("user_api") == "blas"] or [1])
    except Exception:
        blas_threads = 1
    rows = min(rows, L.M)
    t0 = time.perf_counter()
    O.forward_mx(L.A.f32[:rows], L.W.f32, L.q)
    t = time.perf_counter() - t0
    flops = 2.0 * rows * L.N * L.K
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": int(blas_threads),
            "kind": "oracle",
            "sample": f"{rows} of {L.M} rows of A with the full {L.K}x{L.N} W, q={L.q}: the "
                      f"oracle's micro-scaled forward (tau of the sample, clamp + COO, block "
                      f"quantization of A and W, block-scaled float64 product, sparse term) took "
                      f"{t:.2f} s; host affinity {len(os.sched_getaffinity(0))} cpus, BLAS "
                      f"threads {blas_threads}"}


class BackwardStep:
    """The three public calls of one backward GEMM, marshalled once.

    dgrad: dX (M x K) = Q(dY) Q(W)^T, dY and W quantized per row over N.
    wgrad: dW (K x N) = Q(A)^T Q(dY), A and dY quantized per column over M."""

    def __init__(self, ql, which, A, W, dY, stream, mx=False):
        import torch
        lib = ql.lib()
        self.lib, self.which, self.mx = lib, which, mx
        M, K = A.shape
        N = W.shape[1]
        dt = ql.BF16 if A.dtype == torch.bfloat16 else ql.F32
        dev = A.device
        P = ctypes.c_void_p
        self.keep = [A, W, dY]
        self.dt, self.stream = dt, P(stream.cuda_stream)
        if which == "dgrad":
            # operands: dY rows (M x N) and W rows (K x N), both over N
            self.shape = (M, K, N)            # output rows, output cols, reduction
            ops = [(dY, M, N), (W, K, N)]
        else:
            # operands: columns of A (M x K) and of dY (M x N), both over M
            self.shape = (K, N, M)
            ops = [(A, M, K), (dY, M, N)]
        Mo, No, Ko = self.shape
        ldq = ql.packed_ld(Ko)
        nb = ql.mx_scales_ld(Ko)
        self.ops = []
        for X, r, c in ops:
            if mx:
                # micro-scaled: codes plus nb E8M0 bytes per packed row, no workspace
                rows = r if which == "dgrad" else c
                q = torch.empty((rows, ldq), dtype=torch.uint8, device=dev)
                sc = torch.empty((rows * nb,), dtype=torch.uint8, device=dev)
                self.ops.append((P(X.data_ptr()), r, c, X.stride(0), q, sc, None))
            elif which == "dgrad":
                q = torch.empty((r, ldq), dtype=torch.uint8, device=dev)
                sc = torch.empty((r,), dtype=torch.float32, device=dev)
                self.ops.append((P(X.data_ptr()), r, c, X.stride(0), q, sc, None))
            else:
                q = torch.empty((c, ldq), dtype=torch.uint8, device=dev)
                sc = torch.empty((c,), dtype=torch.float32, device=dev)
                wsb = max(int(lib.fp4lin_weight_workspace_bytes(r, c)), 16)
                ws = torch.empty((wsb,), dtype=torch.uint8, device=dev)
                self.ops.append((P(X.data_ptr()), r, c, X.stride(0), q, sc, ws))
        self.out = torch.empty((Mo, No), dtype=torch.float32, device=dev)

    def quant(self, i):
        X, r, c, ld, q, sc, ws = self.ops[i]
        P = ctypes.c_void_p
        if self.mx and self.which == "dgrad":
            st = self.lib.fp4lin_quantize_act_mx(X, self.dt, r, c, ld, None, P(q.data_ptr()),
                                                 P(sc.data_ptr()), self.stream)
        elif self.mx:
            st = self.lib.fp4lin_quantize_weight_mx(X, self.dt, r, c, ld, P(q.data_ptr()),
                                                    P(sc.data_ptr()), self.stream)
        elif self.which == "dgrad":
            st = self.lib.fp4lin_quantize_act(X, self.dt, r, c, ld, None, P(q.data_ptr()),
                                              P(sc.data_ptr()), self.stream)
        else:
            st = self.lib.fp4lin_quantize_weight(X, self.dt, r, c, ld, P(q.data_ptr()),
                                                 P(sc.data_ptr()), P(ws.data_ptr()), ws.numel(),
                                                 self.stream)
        assert st == 0, st

    def gemm(self):
        P = ctypes.c_void_p
        (_, _, _, _, qa, sa, _), (_, _, _, _, qb, sb, _) = self.ops
        Mo, No, Ko = self.shape
        gemm = self.lib.fp4lin_gemm_mx if self.mx else self.lib.fp4lin_gemm
        st = gemm(P(qa.data_ptr()), P(sa.data_ptr()), P(qb.data_ptr()),
                                  P(sb.data_ptr()), Mo, No, Ko, None, None, self.dt, 0,
                                  P(self.out.data_ptr()), No, self.stream)
        assert st == 0, st

    def step(self):
        self.quant(0)
        self.quant(1)
        self.gemm()


def run_backward(args):
    """One JSON line for --pass dgrad / wgrad."""
    import torch
    import quantized_linear_layer_amd as ql
    import workloads as wl
    dev = torch.device("cuda:0")
    L = wl.make_layer(args.workload, seed=args.seed)
    dYh = wl.make_grad_output(L.M, L.N, seed=args.seed)
    A, W, dY = upload(L.A, dev), upload(L.W, dev), upload(dYh, dev)
    stream = torch.cuda.current_stream()
    mx = args.quant == "mx"
    st = BackwardStep(ql, args.which, A, W, dY, stream, mx=mx)
    Mo, No, Ko = st.shape
    flops = 2.0 * Mo * No * Ko
    for _ in range(max(args.warmup, 1)):
        st.step()
    torch.cuda.synchronize()
    f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    f0.record(stream)
    for _ in range(args.steps):
        st.step()
    f1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    event_ms = f0.elapsed_time(f1) / args.steps
    names = ("quant_0", "quant_1", "gemm")
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for i in range(args.steps):
        e = ev[i]
        e[0].record(stream)
        st.quant(0); e[1].record(stream)
        st.quant(1); e[2].record(stream)
        st.gemm(); e[3].record(stream)
    torch.cuda.synchronize()
    stage_ms = {n: float(np.mean([ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(args.steps)]))
                for j, n in enumerate(names)}
    if args.copy_calib:
        copy_calibration(dev)
    gemm_tf = flops / (stage_ms["gemm"] * 1e-3) / 1e12
    e = 2 if L.A.dtype == wl.BF16 else 4
    ldq = ql.packed_ld(Ko)
    # algorithmic bytes of the quantizers: operand read once, codes and scales written
    sbytes = ql.mx_scales_ld(Ko) if mx else 4   # scale bytes per packed row
    qbytes = [e * r * c + (r if args.which == "dgrad" else c) * (ldq + sbytes)
              for (_, r, c, _, _, _, _) in st.ops]
    kernels = {"quant_0": {"ms": round(stage_ms["quant_0"], 5), "bytes": int(qbytes[0]),
                           "GB/s": round(qbytes[0] / (stage_ms["quant_0"] * 1e-3) / 1e9, 1),
                           "bound": "hbm"},
               "quant_1": {"ms": round(stage_ms["quant_1"], 5), "bytes": int(qbytes[1]),
                           "GB/s": round(qbytes[1] / (stage_ms["quant_1"] * 1e-3) / 1e9, 1),
                           "bound": "hbm"},
               "gemm": {"ms": round(stage_ms["gemm"], 5), "TFLOP/s": round(gemm_tf, 1),
                        "mfma_frac": round(gemm_tf / FP4_PEAK_TFLOPS, 4), "bound": "mfma"}}
    traffic = None
    tag = f"{args.workload}_{args.which}" + ("_mx" if mx else "")
    tfile = os.path.join(ROOT, "profiles", f"traffic_gemm_{tag}.json")
    if os.path.exists(tfile):
        tr = json.load(open(tfile))
        if tr.get("source_sha256") == file_sha(os.path.join(ROOT, tr["source"])):
            traffic = tr.get("bytes_per_launch")
    value = flops / (ms_per_step * 1e-3) / 1e12
    what = {"dgrad": "dX = Q(dY) Q(W)^T", "wgrad": "dW = Q(A)^T Q(dY)"}[args.which]
    out = {
        "metric": f"FP4 linear {args.which} effective TFLOP/s ({what}"
                  + (", micro-scaled operands" if mx else "") + ", 1 GPU)",
        "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp4", "data": "synthetic",
        "config": {"workload": tag, "M": L.M, "K": L.K, "N": L.N,
                   "out_rows": Mo, "out_cols": No, "reduction": Ko, "input_dtype": L.A.dtype,
                   "output_dtype": "f32", "seed": args.seed},
        "pct_fp4_peak": round(100.0 * value / FP4_PEAK_TFLOPS, 2),
        "event_ms": round(event_ms, 5),
        "stage_ms": {k: round(v, 5) for k, v in stage_ms.items()},
        "roofline": {"bound": "mfma",
                     "kernel": "fp4_gemm_kernel" + (" (block scales)" if mx else ""),
                     "achieved": round(gemm_tf, 2),
                     "peak": FP4_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(gemm_tf / FP4_PEAK_TFLOPS, 4), "traffic": traffic},
        "kernels": kernels,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_backward(args.which, L, dYh, args.cpu_rows or 64, mx)
    print(json.dumps(out), flush=True)


def cpu_baseline_backward(which, L, dY, rows, mx=False):
    """The oracle's dgrad / wgrad on a sample of output rows (the quantization
    of both whole operands included), timed on the host cores."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()
                            if i.get("user_api") == "blas"] or [1])
    except Exception:
        blas_threads = 1
    nrows = L.M if which == "dgrad" else L.K
    sample = np.arange(min(rows, nrows))
    t0 = time.perf_counter()
    if which == "dgrad":
        (O.dgrad_mx if mx else O.dgrad)(dY.f32, L.W.f32, rows=sample)
        red, cols = L.N, L.K
    else:
        (O.wgrad_mx if mx else O.wgrad)(L.A.f32, dY.f32, rows=sample)
        red, cols = L.M, L.N
    t = time.perf_counter() - t0
    flops = 2.0 * sample.size * cols * red
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": int(blas_threads),
            "kind": "oracle",
            "sample": f"{sample.size} of {nrows} output rows of the {which} GEMM (both operands "
                      f"quantized whole{' in 32-blocks' if mx else ''}, then the float64 "
                      f"{'block-scaled' if mx else 'integer'} product of the sampled rows) "
                      f"took {t:.2f} s; host affinity {len(os.sched_getaffinity(0))} cpus, "
                      f"BLAS threads {blas_threads}"}


STAGES = ("select", "quant_a", "quant_w", "gemm", "sparse")


def cpu_baseline(workload, seed, rows):
    """The oracle as it stands, on the first `rows` rows of the same workload
    (full W), timed on the host cores."""
    import oracle as O
    import workloads as wl
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()
                            if i.get("user_api") == "blas"] or [1])
    except Exception:
        blas_threads = 1
    full = wl.spec(workload)["M"]
    rows = full if rows <= 0 or rows > full else rows
    L = wl.make_layer(workload, seed=seed, M=rows)
    t0 = time.perf_counter()
    Y, _ = O.forward(L.A.f32, L.W.f32, L.q)
    t = time.perf_counter() - t0
    flops = 2.0 * L.M * L.N * L.K
    # the same oracle stages once more, one at a time
    stages = {}

    def timed(name, fn, *a):
        t1 = time.perf_counter()
        r = fn(*a)
        stages[name] = round(time.perf_counter() - t1, 4)
        return r
    tau, _ = timed("rank_and_tau", O.select_threshold, L.A.f32, L.q)
    _, delta = timed("clamp_and_delta", O.clamp_and_residual, L.A.f32, tau)
    _, sA, cA = timed("quantize_a", O.quantize_act, L.A.f32, tau)
    _, sW, cW = timed("quantize_w", O.quantize_weight, L.W.f32)
    acc = timed("integer_gemm", O.integer_product, cA, cW)
    timed("scale_epilogue", O.scaled_product, acc, sA, sW)
    timed("sparse_term", O.sparse_times_dense, delta, L.W.f32)
    del acc
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": int(blas_threads),
            "kind": "oracle", "stages_s": stages,
            "sample": f"{rows} of {full} rows of A with the full {L.K}x{L.N} W, q={L.q}: "
                      f"the whole oracle forward (tau, clamp + COO, quantize A and W, float64 "
                      f"integer GEMM, sparse term) took {t:.2f} s; host affinity "
                      f"{len(os.sched_getaffinity(0))} cpus, BLAS threads {blas_threads}"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); this build has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)
    if args.which != "forward":
        run_backward(args)
        return
    if args.quant == "mx":
        run_forward_mx(args)
        return
    import torch
    import quantized_linear_layer_amd as ql
    import workloads as wl

    dev = torch.device("cuda:0")
    L = wl.make_layer(args.workload, seed=args.seed)
    A = upload(L.A, dev)
    W = upload(L.W, dev)
    stream = torch.cuda.current_stream()
    st = Step(ql, A, W, L.q, stream)
    M, K, N = L.M, L.K, L.N
    flops = 2.0 * M * N * K

    # warmup (also checks the path end to end once)
    for _ in range(max(args.warmup, 1)):
        st.select(); st.quant_a(); st.quant_w(); st.gemm(); st.sparse()
        st.forward_call()
    torch.cuda.synchronize()
    nnz = int(st.ws[st.offsets.row_ptr + 4 * M: st.offsets.row_ptr + 4 * M + 4]
              .cpu().numpy().view(np.int32)[0])

    # timed region: exactly K steps, one fp4lin_forward call each
    f0 = torch.cuda.Event(enable_timing=True)
    f1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    f0.record(stream)
    for _ in range(args.steps):
        st.forward_call()
    f1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    forward_event_ms = f0.elapsed_time(f1) / args.steps

    # secondary: the forward with the caches behind L2 cold (512 MB written
    # before each call, outside the events)
    flush = torch.empty(1 << 27, dtype=torch.float32, device=dev)
    cold = []
    for _ in range(min(args.steps, 20)):
        flush.zero_()
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        st.forward_call()
        c1.record(stream)
        torch.cuda.synchronize()
        cold.append(c0.elapsed_time(c1))
    del flush
    forward_cold_ms = float(np.median(cold))

    # breakdown: the same work as separate public calls, events between stages
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(STAGES) + 1)]
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        e = ev[i]
        e[0].record(stream)
        st.select(); e[1].record(stream)
        st.quant_a(); e[2].record(stream)
        st.quant_w(); e[3].record(stream)
        st.gemm(); e[4].record(stream)
        st.sparse(); e[5].record(stream)
    torch.cuda.synchronize()
    stage_ms = {name: float(np.mean([ev[i][j].elapsed_time(ev[i][j + 1])
                                     for i in range(args.steps)]))
                for j, name in enumerate(STAGES)}
    stages_step_ms = float(np.mean([ev[i][0].elapsed_time(ev[i][-1]) for i in range(args.steps)]))

    if args.copy_calib:
        copy_calibration(dev)

    value = flops / (ms_per_step * 1e-3) / 1e12
    # Algorithmic work per launch of each stage (the minimum the operation
    # needs; the roofline each stage is held against):
    #   select  : A read twice (threshold, then compaction) + COO + row_ptr written
    #   quant_a : A read once, packed codes + scales written
    #   quant_w : W read once, packed codes + scales written
    #   gemm    : 2*M*N*K FP4 MFMA flops (its HBM floor, packed operands read
    #             once + fp32 Y written, is below the MFMA floor)
    #   sparse  : Y read and written, COO read, each touched W row read once
    e = 2 if L.A.dtype == wl.BF16 else 4
    ldq = ql.packed_ld(K)
    hbm_bytes = {
        "select": 2 * e * M * K + 12 * nnz + 4 * (M + 1),
        "quant_a": e * M * K + M * ldq + 4 * M,
        "quant_w": e * K * N + N * ldq + 4 * N,
        "gemm": (M + N) * ldq + 4 * M * N,
        "sparse": 8 * M * N + 12 * nnz + 4 * (M + 1) + e * N * min(K, nnz),
    }
    kernels = {}
    for name in STAGES:
        t_s = stage_ms[name] * 1e-3
        gbs = hbm_bytes[name] / t_s / 1e9
        kernels[name] = {"ms": round(stage_ms[name], 5), "bytes": int(hbm_bytes[name]),
                         "GB/s": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
    gemm_tf = flops / (stage_ms["gemm"] * 1e-3) / 1e12
    kernels["gemm"].update({"bound": "mfma", "TFLOP/s": round(gemm_tf, 1),
                            "mfma_frac": round(gemm_tf / FP4_PEAK_TFLOPS, 4)})
    # the compensation is 2*nnz*N fp32 flop on the vector ALUs (one FMA per
    # non-zero and output column); its HBM bytes are far below its ALU time
    sp_flops = 2.0 * nnz * N
    sp_tf = sp_flops / (stage_ms["sparse"] * 1e-3) / 1e12
    kernels["sparse"].update({"bound": "alu", "fp32_TFLOP/s": round(sp_tf, 2),
                              "alu_frac": round(sp_tf / VALU_FP32_PEAK_TFLOPS, 4)})
    for name in ("select", "quant_a", "quant_w"):
        kernels[name]["bound"] = "hbm"
    dom = max(STAGES, key=lambda n: stage_ms[n])
    traffic = None
    tfile = os.path.join(ROOT, "profiles", f"traffic_{dom}_{args.workload}.json")
    if os.path.exists(tfile):
        tr = json.load(open(tfile))
        if tr.get("source_sha256") == file_sha(os.path.join(ROOT, tr["source"])):
            traffic = tr.get("bytes_per_launch")
    if dom == "gemm":
        roof = {"bound": "mfma", "kernel": "fp4_gemm_kernel", "achieved": round(gemm_tf, 2),
                "peak": FP4_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(gemm_tf / FP4_PEAK_TFLOPS, 4),
                "traffic": traffic}
    elif dom == "sparse":
        roof = {"bound": "alu", "kernel": "sparse_add_kernel", "achieved": round(sp_tf, 2),
                "peak": VALU_FP32_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(sp_tf / VALU_FP32_PEAK_TFLOPS, 4), "traffic": traffic}
    else:
        kname = {"select": "select_hist/count/compact kernels", "quant_a": "quantize_rows_kernel",
                 "quant_w": "colmax + quantize_cols kernels"}[dom]
        roof = {"bound": "hbm", "kernel": kname, "achieved": kernels[dom]["GB/s"],
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": kernels[dom]["hbm_frac"],
                "traffic": traffic}
    # algorithmic HBM bytes of the whole forward (A read twice, W read once,
    # packed operands written and read once, Y written once, COO written/read)
    alg_bytes = (2 * e * M * K + e * K * N + 2 * (M + N) * ldq + 4 * M * N + 2 * 12 * nnz)
    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4",
        "data": "synthetic",
        "config": {"workload": args.workload, "M": M, "K": K, "N": N, "q": L.q,
                   "input_dtype": L.A.dtype, "output_dtype": "f32", "seed": args.seed,
                   "nnz_dA": nnz},
        "pct_fp4_peak": round(100.0 * value / FP4_PEAK_TFLOPS, 2),
        "pct_hbm_roofline": round(100.0 * (alg_bytes / (ms_per_step * 1e-3) / 1e9) / HBM_PEAK_GBS, 2),
        "forward_event_ms": round(forward_event_ms, 5),
        "forward_cold_ms": round(forward_cold_ms, 5),
        "stage_ms": {k: round(v, 5) for k, v in stage_ms.items()},
        "stages_step_ms": round(stages_step_ms, 5),
        "roofline": roof,
        "kernels": kernels,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.workload, args.seed, args.cpu_rows)
    if args.workload == "llama7b_ffn_up" and not args.no_13b:
        # the 13B FFN shapes beside the 7B headline (one layer at a time)
        del st, A, W
        torch.cuda.empty_cache()
        up, down = wl.make_13b_pair(seed=args.seed)
        n13 = max(1, min(args.steps, 10))
        # 20 untimed calls first: the GPU sat idle during the CPU baseline, and
        # its clock needs some milliseconds of load to come back up
        out["llama13b_ffn_up"] = forward_rate(up, dev, n13, 20)
        del up
        torch.cuda.empty_cache()
        out["llama13b_ffn_down"] = forward_rate(down, dev, n13, 20)
        del down
        torch.cuda.empty_cache()
    print(json.dumps(out), flush=True)


def copy_calibration(dev):
    """Plain copies of known size for PMC byte calibration: 1 GiB read and
    1 GiB written, by the runtime's blit kernel and by an elementwise kernel."""
    import torch
    src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    del src, dst


def upload(m, dev):
    import torch
    import workloads as wl
    if m.dtype == wl.F32:
        return torch.from_numpy(np.ascontiguousarray(m.bits)).to(dev)
    return torch.from_numpy(np.ascontiguousarray(m.bits).view(np.int16)).to(dev).view(torch.bfloat16)

if __name__ == "__main__":
    main()
