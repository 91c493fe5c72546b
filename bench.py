#!/usr/bin/env python3
"""Benchmark of the fused-chain hot path on one MI355X.

One step = one pass of every hot-path row over one batch of synthetic input:
  chain    n = 16,777,216 fp32, K in {2,3,4,6,8}: naive (K launches, ping-pong)
           and fused (1 launch); fat probe at K = 4 with 48 live fp32x4 temps;
           8-stage affine chain h <- 1.01 h + 0.01 on 1,048,576 elements, fused
           vs 8 single-stage launches
  decode   GEMM + bias + GELU + residual at M = 16, N = K = 4096, four plans
  gemm     Y = GELU(A.B + bias) + R at M = N = K = 4096 fp16, plans
           [1,1,1,1], [1,3], [2,2], [4]
  softmax  causal scaled softmax over [8,16,2048,2048] bf16: fused with tile
           64/128/256 and without skipping, plus the unfused five-step
           baseline with its mask materialisation

`value` is the fused path's HBM throughput: algorithmic bytes of the fused
chain (all K) and the fused softmax (tile 64) divided by their summed kernel
time.  Kernel times come from HIP events recorded on the stream the kernels are
launched on.  HBM rows rotate over several buffer sets so repeats cannot be
served from the 256 MiB MALL.

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fused-chain/softmax HBM GB/s (% peak); GEMM+epilogue TFLOP/s at 4096³ fp16"
HBM_PEAK_GBPS = 8000.0
FP16_PEAK_TFLOPS = 2500.0

CHAIN_N = 16777216
CHAIN_KS = [2, 3, 4, 6, 8]
CHAIN_SETS = 5                      # 5 x 128 MiB touched per rotation
FAT_K, FAT_T = 4, 48
AFFINE_N, AFFINE_K = 1048576, 8
AFFINE_SETS = 40                    # 40 x 8 MiB touched per rotation (beyond the MALL)
DECODE_MNK = (16, 4096, 4096)
DECODE_SETS = 17                    # 17 copies of the 32 MiB weight matrix: ceil(512 MiB / footprint) + 1
GEMM_MNK = (4096, 4096, 4096)
PLANS = [[1, 1, 1, 1], [1, 3], [2, 2], [4]]
SM_B, SM_H, SM_S = 8, 16, 2048
SM_TILES = [64, 128, 256, 2048]
SCALE = 1.0 / (128.0 ** 0.5)
ATT_BH, ATT_S, ATT_D = SM_B * SM_H, SM_S, 128   # attention over the softmax workload's heads and length
RMS_ROWS, RMS_D, RMS_EPS = 1024, 4096, 1e-5     # n = 4,194,304 fp32 (the ledger's ~4M), rows of d_model 4096
RMS_SETS = 17                                    # 17 x 32 MiB: ceil(512 MiB / footprint) + 1
MIN_ROW_SAMPLES = 50                             # event pairs per row at least


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class Timer:
    """Event pairs on the launch stream; elapsed times collected per row.

    A row is `reps` calls of the binding, launched from the host as they come
    (the host runs ahead of the GPU, so kernels follow each other without
    gaps).  With graph=True the first run of a row runs its calls once eagerly,
    then captures them into a HIP graph, and from then on the row is one graph
    replay between the two
    events; on this stack that adds one to two microseconds per kernel node, so
    it is not the default."""

    def __init__(self, torch, stream, graph=False):
        self.torch, self.stream, self.eager = torch, stream, not graph
        self.pending = []
        self.ms = {}
        self.graphs = {}

    def __call__(self, name, fn, reps=1):
        t = self.torch
        g = None
        if not self.eager:
            g = self.graphs.get(name)
            if g is None:
                # one eager run first: library handles (the vendor GEMM's among
                # them) initialise outside the capture
                for r in range(reps):
                    fn(r)
                t.cuda.synchronize()
                g = t.cuda.CUDAGraph()
                with t.cuda.graph(g):
                    for r in range(reps):
                        fn(r)
                self.graphs[name] = g
        e0 = t.cuda.Event(enable_timing=True)
        e1 = t.cuda.Event(enable_timing=True)
        e0.record(self.stream)
        if g is not None:
            g.replay()
        else:
            for r in range(reps):
                fn(r)
        e1.record(self.stream)
        self.pending.append((name, e0, e1, reps))

    def collect(self):
        for name, e0, e1, reps in self.pending:
            self.ms.setdefault(name, []).append(e0.elapsed_time(e1) / reps)
        self.pending = []

    def median(self, name):
        v = sorted(self.ms[name])
        return v[len(v) // 2]

    def minimum(self, name):
        return min(self.ms[name])


def source_hash(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def load_traffic(kernel_key, src):
    """HBM traffic per launch measured with rocprofv3 counters, if the kernel
    source is unchanged since the counters were taken."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        tab = json.load(f)
    row = tab.get(kernel_key)
    if not row or row.get("source_sha") != source_hash(src):
        return None
    return row.get("bytes_per_launch")


def oracle_stream_rate(budget_s, heads_per_pass=16):
    """Algorithmic GB/s of the oracle on whole passes of the fused chain (K in
    {2,3,4,6,8}, n = 16,777,216) and of the causal softmax over [2048, 2048]
    heads, repeated until about `budget_s` seconds of host work.  Returns
    (GB/s, chain passes, chain seconds, heads, softmax seconds)."""
    import numpy as np

    import oracle
    import synth
    from oracle import ledger

    n = CHAIN_N
    x, _, _ = synth.chain_inputs(n, 1)
    coefs = [synth.chain_inputs(1, K)[1:] for K in CHAIN_KS]
    S = SM_S
    s = synth.softmax_inputs(1, S, salt=11)
    rows = np.arange(S)
    chain_passes = heads = 0
    t_chain = t_sm = 0.0
    while t_chain + t_sm < budget_s:
        t0 = time.perf_counter()
        for a, b in coefs:
            oracle.chain_f64(x, a, b, True)
        t_chain += time.perf_counter() - t0
        chain_passes += 1
        t0 = time.perf_counter()
        for _ in range(heads_per_pass):
            oracle.causal_softmax_rows(s, SCALE, rows)
        t_sm += time.perf_counter() - t0
        heads += heads_per_pass
    chain_bytes = chain_passes * sum(ledger.chain_bytes(n, K, True) for K in CHAIN_KS)
    sm_bytes = heads * ledger.softmax_bytes(1, S, 64, True)
    return (chain_bytes + sm_bytes) / (t_chain + t_sm) / 1e9, chain_passes, t_chain, heads, t_sm


def _oracle_single_thread(budget_s=4.0):
    """The same stream sample on one host thread, in a child process (the
    oracle's OpenMP pool is sized when it starts; the child touches no GPU)."""
    import subprocess
    code = ("import json, sys; sys.path.insert(0, %r); import bench; "
            "r = bench.oracle_stream_rate(%r, heads_per_pass=2); print(json.dumps(r))") % (ROOT, budget_s)
    env = dict(os.environ, OMP_NUM_THREADS="1")
    try:
        out = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120,
                             check=True).stdout.strip().splitlines()[-1]
        gbps, passes, t_c, heads, t_s = json.loads(out)
    except Exception as e:                      # reported, never fatal to the GPU measurement
        return {"error": f"{type(e).__name__}: {e}"[:200]}
    return {"value": round(gbps, 3), "unit": "GB/s", "cores": 1,
            "sample": f"{passes} chain pass(es) ({t_c:.1f}s) and {heads} softmax heads ({t_s:.1f}s) on one thread"}


def _host_cpu():
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "model": model}


def cpu_baseline(budget_s=12.0):
    """The oracle, as it stands, on a bounded sample of the same workload:
    whole passes of the fused chain and of the causal softmax (see
    oracle_stream_rate) for about `budget_s` seconds on the host's OpenMP
    threads, and the same sample on one thread; reported in the same unit
    (algorithmic GB/s).  The GEMM epilogue is timed on sampled outputs of the
    4096^3 chain, attention on every query row of 8 heads."""
    import numpy as np

    import oracle
    import synth

    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    gbps, chain_passes, t_chain, heads, t_sm = oracle_stream_rate(budget_s)
    M, N, K = GEMM_MNK
    A, B, bias, R = synth.gemm_inputs(M, N, K)
    cnt = 262144
    rr = np.random.default_rng(0)
    t0 = time.perf_counter()
    oracle.gemm_epilogue_at(A, B, bias, R, rr.integers(0, M, cnt), rr.integers(0, N, cnt))
    t_g = time.perf_counter() - t0
    tflops = 2.0 * K * cnt / t_g / 1e12
    # attention: every query row of 8 [2048, 128] heads (the oracle's cost of
    # a row grows with its causal prefix)
    att_heads = 8
    Qa, Ka, Va = synth.attention_inputs(att_heads, ATT_S, ATT_D, salt=11)
    t0 = time.perf_counter()
    oracle.causal_attention_rows(Qa, Ka, Va, SCALE, np.arange(att_heads * ATT_S))
    t_a = time.perf_counter() - t0
    att_tflops = 2.0 * ATT_D * ATT_S * (ATT_S + 1) * att_heads / t_a / 1e12
    return {
        "value": round(gbps, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
        "sample": (f"fp64 C oracle on {threads} threads: {chain_passes} pass(es) of the fused chain K in "
                   f"{CHAIN_KS} over n=16,777,216 ({t_chain:.1f}s) and {heads} causal-softmax heads of "
                   f"[2048, 2048] (one synthetic head repeated; {t_sm:.1f}s); bytes counted as the fused "
                   f"kernels' algorithmic bytes for the same work"),
        "gemm_epilogue": {"value": round(tflops, 6), "unit": "TFLOP/s",
                          "sample": f"{cnt} sampled outputs of the 4096^3 chain (2*K flops each) in {t_g:.1f}s"},
        "attention": {"value": round(att_tflops, 6), "unit": "TFLOP/s",
                      "sample": f"all query rows of {att_heads} [2048, 128] heads (causal flops) in {t_a:.1f}s"},
        "single_thread": _oracle_single_thread(),
        "host": _host_cpu(),
    }


def _fail(msg):
    log(f"PARITY FAILURE: {msg}")
    raise SystemExit(3)


def cpu_baseline_leg_parity(torch, fc, groups, bufs):
    """First part of the cpu_baseline leg, run before the warmup: the oracle on
    the host computes reference values for outputs of every row on the bench's
    own resident inputs (set 0), each row runs once on the GPU, and the results
    must meet the parity tests' bars, else the run stops (exit status 3):
      chain    fused / naive (every K) and fat (K = 4, T = 48) y equal to the
               one-rounding fp32 chain and within 1e-6 normwise of the fp64 one;
               the fat sink equal to its fp32 formula; byte ledgers equal;
      affine   fused / naive within 1e-6 normwise of the collapsed closed form;
      decode   every output of every plan within 1e-2 (1 + |ref|);
      gemm     4,096 sampled outputs (tile corners included) of every plan, same bar;
      softmax  64 sampled rows of every tile and of the unfused form within 1e-2,
               exact zeros above the diagonal, row sums within 1e-3 plus half a
               bf16 ulp per entry; byte ledgers equal;
      attention 64 sampled rows within 2^-8 (|ref| + max_{j<=i} |V|);
      rmsnorm  16 sampled rows of both forms within 4e-6 |ref|.
    Returns a summary (the worst error over its bar per row, <= 1) and the
    affine row's closed-form errors and oracle time."""
    import numpy as np

    import oracle
    from oracle import ledger

    out, extra = {}, {}
    rr = np.random.default_rng(123)

    def host(t):
        return t.detach().cpu().numpy()

    def hbits(t):
        return t.view(torch.int16).cpu().numpy().view(np.uint16)

    def f16v(b):
        return b.view(np.float16).astype(np.float64)

    def bf16v(b):
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)

    def normwise(y, ref):
        return float(np.max(np.abs(np.asarray(y, np.float64) - ref)) / max(np.max(np.abs(ref)), 1e-300))

    if "chain" in groups:
        sets, coef = bufs["chain"]
        x = host(sets[0][0])
        worst = 0.0
        y = torch.empty_like(sets[0][0])
        for K in CHAIN_KS:
            a, b = coef[K]
            if fc.fc_chain_bytes(CHAIN_N, K, fc.FC_CHAIN_FUSED) != ledger.chain_bytes(CHAIN_N, K, True) or \
                    fc.fc_chain_bytes(CHAIN_N, K, fc.FC_CHAIN_NAIVE) != ledger.chain_bytes(CHAIN_N, K, False):
                _fail(f"chain K={K}: byte ledger")
            ref32 = oracle.chain_f32fma(x, a, b, True)
            ref64 = oracle.chain_f64(x, a, b, True)
            for mode in (fc.FC_CHAIN_FUSED, fc.FC_CHAIN_NAIVE):
                fc.fc_chain(sets[0][0], y, a, b, True, mode, sets[0][2])
                yh = host(y)
                if not np.array_equal(yh, ref32):
                    _fail(f"chain K={K} mode={mode}: differs from the one-rounding fp32 oracle")
                e = normwise(yh, ref64)
                if e > 1e-6:
                    _fail(f"chain K={K} mode={mode}: normwise {e}")
                worst = max(worst, e / 1e-6)
        a, b = coef[FAT_K]
        sink = bufs["chain_sink"]
        fc.fc_chain(sets[0][0], y, a, b, True, fc.FC_CHAIN_FAT, sink, FAT_T)
        if not np.array_equal(host(y), oracle.chain_f32fma(x, a, b, True)):
            _fail("fat probe: y differs from the oracle")
        if not np.array_equal(host(sink), oracle.chain_fat_sink_f32(x, a, b, True, FAT_T, sink.numel() // 4)):
            _fail("fat probe: sink differs from its formula")
        out["chain"] = {"checked": f"every element of fused and naive (K in {CHAIN_KS}) and fat K={FAT_K} "
                                   f"T={FAT_T} (y and sink)", "worst_over_bar": round(worst, 4)}
    if "affine" in groups:
        asets, aa, ab = bufs["affine"]
        x = host(asets[0][0]).astype(np.float64)
        from fractions import Fraction
        A, B = Fraction(float(aa[0])), Fraction(float(ab[0]))
        closed = x * float(A ** AFFINE_K) + float(B * (A ** AFFINE_K - 1) / (A - 1))
        y = torch.empty_like(asets[0][0])
        errs = {}
        for mode, nm in ((fc.FC_CHAIN_FUSED, "fused"), (fc.FC_CHAIN_NAIVE, "naive")):
            fc.fc_chain(asets[0][0], y, aa, ab, False, mode, asets[0][2])
            errs[nm] = normwise(host(y), closed)
            if errs[nm] > 1e-6:
                _fail(f"affine {nm}: normwise {errs[nm]} against the closed form")
        xf = host(asets[0][0])
        ts = []
        for _ in range(3):
            t0 = time.perf_counter()
            oracle.chain_f64(xf, aa, ab, False)
            ts.append(time.perf_counter() - t0)
        extra["affine"] = {"closed_form_normwise_err_fused": errs["fused"],
                           "closed_form_normwise_err_naive": errs["naive"],
                           "oracle_fp64_ms": round(sorted(ts)[1] * 1e3, 3),
                           "oracle_threads": int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))}
        out["affine"] = {"checked": "every element, fused and 8 launches, against the collapsed form",
                         "worst_over_bar": round(max(errs.values()) / 1e-6, 4)}
    if "decode" in groups:
        d0 = bufs["decode"][0]
        h = [hbits(t) for t in d0[:4]]
        ref = oracle.gemm_epilogue_f64_matmul(*h)
        worst = 0.0
        for plan in PLANS:
            Y = torch.empty_like(d0[4])
            fc.fc_gemm_epilogue(*d0[:4], Y, plan, d0[5])
            r = float(np.max(np.abs(f16v(hbits(Y)) - ref) / (1e-2 * (1 + np.abs(ref)))))
            if not r <= 1.0:
                _fail(f"decode plan {plan}: {r} of the bar")
            worst = max(worst, r)
        out["decode"] = {"checked": "every output of every plan", "worst_over_bar": round(worst, 4)}
    if "gemm" in groups:
        A, B, bias, R = bufs["gemm"]
        Y, ws = bufs["gemm_out"]
        h = [hbits(t) for t in (A, B, bias, R)]
        M, N, K = GEMM_MNK
        rows = np.concatenate([rr.integers(0, M, 4088), [0, 0, M - 1, M - 1, 255, 256, 255, 256]])
        cols = np.concatenate([rr.integers(0, N, 4088), [0, N - 1, 0, N - 1, 255, 256, 256, 255]])
        for plan in PLANS:
            if fc.fc_plan_bytes(M, N, K, plan) != ledger.plan_bytes(M, N, K, plan):
                _fail(f"gemm plan {plan}: byte ledger")
        ref = oracle.gemm_epilogue_at(*h, rows, cols)
        worst = 0.0
        for plan in PLANS:
            fc.fc_gemm_epilogue(A, B, bias, R, Y, plan, ws)
            y = f16v(hbits(Y)[rows, cols])
            r = float(np.max(np.abs(y - ref) / (1e-2 * (1 + np.abs(ref)))))
            if not r <= 1.0:
                _fail(f"gemm plan {plan}: {r} of the bar")
            worst = max(worst, r)
        out["gemm"] = {"checked": "4,096 sampled outputs of every plan", "worst_over_bar": round(worst, 4)}
    if "softmax" in groups:
        sd, so = bufs["softmax"]
        smws = bufs["softmax_ws"]
        BH, S = SM_B * SM_H, SM_S
        rows = np.unique(np.concatenate([rr.integers(0, BH * S, 56), [0, 1, 63, 64, 2047, 2048, 4095, BH * S - 1]]))
        rid = torch.from_numpy(rows).to(sd.device)
        ref = oracle.causal_softmax_rows(hbits(sd), SCALE, rows)
        for tile in SM_TILES:
            if fc.fc_softmax_bytes(BH, S, tile, fc.FC_SOFTMAX_FUSED) != ledger.softmax_bytes(BH, S, tile, True):
                _fail(f"softmax tile {tile}: byte ledger")
        runs = [(f"fused_T{t}", lambda t=t: fc.fc_causal_softmax(sd, so, SCALE, t, fc.FC_SOFTMAX_FUSED))
                for t in SM_TILES]
        runs.append(("unfused", lambda: (fc.fc_causal_mask_materialise(smws, BH, S),
                                         fc.fc_causal_softmax(sd, so, SCALE, 64, fc.FC_SOFTMAX_UNFUSED, smws))))
        worst = 0.0
        i = rows % S
        kept = np.arange(S)[None, :] <= i[:, None]
        for nm, run in runs:
            run()
            o = bf16v(hbits(so.view(BH * S, S)[rid]))
            err = float(np.max(np.abs(o - ref)))
            if err > 1e-2 or np.any(o[~kept] != 0) or not np.all(o[kept] > 0):
                _fail(f"softmax {nm}: error {err} or zero pattern")
            e = np.floor(np.log2(np.where(o > 0, o, 1.0)))
            slack = 1e-3 + np.where(o > 0, 2.0 ** (e - 8), 0.0).sum(1)
            if np.any(np.abs(o.sum(1) - 1.0) > slack):
                _fail(f"softmax {nm}: a row sum beyond its bar")
            worst = max(worst, err / 1e-2)
        out["softmax"] = {"checked": f"{rows.size} sampled rows of every tile and of the unfused form",
                          "worst_over_bar": round(worst, 4)}
    if "attention" in groups:
        qa, ka, va, _ = bufs["attention"]
        BH, S, D = ATT_BH, ATT_S, ATT_D
        rows = np.unique(np.concatenate([rr.integers(0, BH * S, 58), [0, 1, 127, 128, 2047, BH * S - 1]]))
        Q, Kh, V = hbits(qa), hbits(ka), hbits(va)
        ref = oracle.causal_attention_rows(Q, Kh, V, SCALE, rows)
        o = torch.empty_like(qa)
        fc.fc_causal_attention(qa, ka, va, o, SCALE)
        got = bf16v(hbits(o).reshape(BH * S, D)[rows])
        vabs = np.abs(bf16v(V))
        bound_v = np.stack([vabs[r // S, : r % S + 1].max(0) for r in rows])
        ratio = float(np.max(np.abs(got - ref) / (2.0 ** -8 * (np.abs(ref) + bound_v))))
        if not ratio <= 1.0:
            _fail(f"attention: {ratio} of the bar")
        out["attention"] = {"checked": f"{rows.size} sampled query rows", "worst_over_bar": round(ratio, 4)}
    if "rmsnorm" in groups:
        rsets, grms = bufs["rmsnorm"]
        rws = bufs["rmsnorm_ws"]
        rows = np.unique(np.concatenate([rr.integers(0, RMS_ROWS, 14), [0, RMS_ROWS - 1]]))
        x = host(rsets[0][0])[rows]
        ref = oracle.rmsnorm_f64(x, host(grms), RMS_EPS)
        worst = 0.0
        for mode in (fc.FC_RMSNORM_FUSED, fc.FC_RMSNORM_UNFUSED):
            y = torch.empty_like(rsets[0][0])
            fc.fc_rmsnorm(rsets[0][0], grms, y, RMS_EPS, mode, rws)
            r = float(np.max(np.abs(host(y)[rows] - ref) / (4e-6 * np.abs(ref) + 1e-300)))
            if not r <= 1.0:
                _fail(f"rmsnorm mode {mode}: {r} of the bar")
            worst = max(worst, r)
        out["rmsnorm"] = {"checked": f"{rows.size} sampled rows of both forms", "worst_over_bar": round(worst, 4)}
    torch.cuda.synchronize()
    return out, extra


def measure_model_rows(torch, stream, groups, bufs, fc):
    """Inputs of the split-plan cost model on this device and the rows that
    validate it: the per-launch cost of a stream (back-to-back empty kernels),
    a t(n) = a + b n fit of plain copies, the fat probe's register sweep, and
    every split plan of both GEMM shapes (eager, and for the decode shape also
    replayed from a captured HIP graph)."""
    from gemm_epilogues_amd import envelope as env
    dev = torch.device("cuda", 0)
    out = {}
    sink = torch.zeros(64, dtype=torch.float32, device=dev)
    n_l = 200
    # per-kernel cost on the device's timeline: n_l empty kernels enqueued by
    # one host call (as one library call enqueues the kernels of a split plan)
    ms = _median_ms(torch, stream, lambda r: env.fce_empty_n(256, n_l, sink), 1, iters=9) / n_l
    out["launch_us"] = round(ms * 1e3, 3)
    # the same kernel with one binding call per launch: the host's pace
    ms = _median_ms(torch, stream, lambda r: env.fce_empty(256, sink), n_l, iters=9)
    out["host_call_us"] = round(ms * 1e3, 3)
    # t(n) for plain copies of n bytes (read n + write n), enqueued `reps` at a
    # time by one host call; least-squares a + b * 2n
    big = torch.empty(2 * (256 << 20), dtype=torch.uint8, device=dev)
    src, dst = big[: 256 << 20], big[256 << 20:]
    pts = []
    for nb in (32 << 10, 256 << 10, 2 << 20, 16 << 20, 64 << 20, 256 << 20):
        reps = 50 if nb <= (2 << 20) else 10
        t = _median_ms(torch, stream, lambda r, nb=nb, reps=reps: env.fce_mix_n(src, nb, dst, nb, reps), 1,
                       iters=7) * 1e-3 / reps
        pts.append((2 * nb, t))
    xs = [p[0] for p in pts]
    ys = [p[1] for p in pts]
    mx, my = sum(xs) / len(xs), sum(ys) / len(ys)
    b = sum((x - mx) * (y - my) for x, y in zip(xs, ys)) / sum((x - mx) ** 2 for x in xs)
    a = my - b * mx
    out["copy_t_of_n"] = {"points": [{"bytes": x, "us": round(y * 1e6, 2)} for x, y in pts],
                          "a_us": round(a * 1e6, 2), "GBps_from_b": round(1.0 / b / 1e9, 1)}
    del big, src, dst
    if "chain" in groups:
        sets, coef = bufs["chain"]
        a4, b4 = synth_chain_coef(4)
        sweep = []
        t_fused = _median_ms(torch, stream, lambda r: fc.fc_chain(sets[r][0], sets[r][1], a4, b4, True,
                                                                     fc.FC_CHAIN_FUSED), CHAIN_SETS)
        for T in (0, 16, 48, 96, 128):
            sk = torch.empty(fc.fc_chain_scratch_floats(CHAIN_N, 4, fc.FC_CHAIN_FAT, T), dtype=torch.float32,
                             device=dev)
            t = _median_ms(torch, stream, lambda r, T=T, sk=sk: fc.fc_chain(sets[r][0], sets[r][1], a4, b4, True,
                                                                             fc.FC_CHAIN_FAT, sk, T), CHAIN_SETS)
            r = fc.fc_kernel_info(f"fc::chain_fat_kernel<4, true, {T}>")
            sweep.append({"T": T, "us": round(t * 1e3, 2), "over_fused": round(t / t_fused, 2),
                          "vgprs": r["vgprs"], "agprs": r["agprs"], "waves_per_simd": r["waves_per_simd"],
                          "scratch_bytes_per_lane": r["scratch_bytes"]})
        out["fat_sweep_K4"] = {"fused_us": round(t_fused * 1e3, 2), "rows": sweep}
    plans_all = [[4], [3, 1], [1, 3], [2, 2], [2, 1, 1], [1, 2, 1], [1, 1, 2], [1, 1, 1, 1]]
    meas = {}
    if "decode" in groups:
        dsets = bufs["decode"]
        M, N, K = DECODE_MNK
        rows = {}
        for plan in plans_all:
            t = _median_ms(torch, stream, lambda r, plan=plan: fc.fc_gemm_epilogue(*dsets[r][:5], plan, dsets[r][5]),
                           DECODE_SETS)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for r in range(DECODE_SETS):
                    fc.fc_gemm_epilogue(*dsets[r][:5], plan, dsets[r][5])
            tg = _median_ms(torch, stream, lambda r, g=g: g.replay(), 1) / DECODE_SETS
            rows["".join(map(str, plan))] = {"us": round(t * 1e3, 2), "graph_replay_us": round(tg * 1e3, 2)}
            meas[("decode", tuple(plan))] = t * 1e-3
        out["decode_all_plans"] = rows
    if "gemm" in groups and "gemm_out" in bufs:
        A, B, bias, R = bufs["gemm"]
        Y, ws = bufs["gemm_out"]
        rows = {}
        for plan in plans_all:
            t = _median_ms(torch, stream, lambda r, plan=plan: fc.fc_gemm_epilogue(A, B, bias, R, Y, plan, ws), 1,
                           iters=9)
            rows["".join(map(str, plan))] = {"us": round(t * 1e3, 2)}
            meas[("gemm", tuple(plan))] = t * 1e-3
        out["gemm4096_all_plans"] = rows
    out["_measured"] = meas
    torch.cuda.synchronize()
    return out


def synth_chain_coef(K):
    import synth
    return synth.chain_inputs(1, K)[1:]


def _median_ms(torch, stream, fn, reps, iters=7):
    """Median over `iters` event pairs of the time per call of `reps` calls."""
    ts = []
    for _ in range(iters):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for r in range(reps):
            fn(r)
        e1.record(stream)
        e1.synchronize()
        ts.append(e0.elapsed_time(e1) / reps)
    ts.sort()
    return ts[len(ts) // 2]


def measure_references(torch, stream, groups, bufs, fc):
    """Reachable reference rates for each row's traffic mix on this device
    (libfcenv.so probes: plain streams and a plain MFMA loop), on the rows' own
    cold buffers.  A fraction of 1 or more means the kernel moves its bytes at
    least as fast as a plain stream of the same mix."""
    from gemm_epilogues_amd import envelope as env
    C = env.fce_chunk_bytes()
    dev = torch.device("cuda", 0)
    out = {}
    for _ in range(2):                         # first pass warms the probes up
        if "chain" in groups:
            sets, _ = bufs["chain"]
            nb = CHAIN_N * 4
            ms = _median_ms(torch, stream, lambda r: env.fce_mix(sets[r][0], nb, sets[r][1], nb), CHAIN_SETS)
            out["copy_64MiB_cold"] = {"GBps": round(2 * nb / ms / 1e6, 1), "bytes": 2 * nb,
                                      "probe": "fce_mix read 64 MiB + write 64 MiB, 5 rotating sets"}
        if "softmax" in groups:
            sd, so = bufs["softmax"]
            W = sd.numel() * 2
            for tile in (64, 2048):
                rb = fc.fc_softmax_bytes(SM_B * SM_H, SM_S, tile, fc.FC_SOFTMAX_FUSED) - W
                rb -= rb % C
                ms = _median_ms(torch, stream, lambda r, rb=rb: env.fce_mix(sd, rb, so, W), 1)
                out[f"mix_softmax_T{tile}"] = {"GBps": round((rb + W) / ms / 1e6, 1), "read_bytes": rb,
                                               "write_bytes": W,
                                               "probe": "fce_mix with the row's read/write byte mix"}
        if "decode" in groups:
            dsets = bufs["decode"]
            nb = dsets[0][1].numel() * 2
            sink = torch.zeros(1, dtype=torch.float32, device=dev)
            ms = _median_ms(torch, stream, lambda r: env.fce_read(dsets[r][1], nb, sink), DECODE_SETS)
            out["read_32MiB_cold"] = {"GBps": round(nb / ms / 1e6, 1), "bytes": nb,
                                      "probe": f"fce_read of B, {DECODE_SETS} rotating copies"}
        if "rmsnorm" in groups:
            rsets, _ = bufs["rmsnorm"]
            nb = rsets[0][0].numel() * 4
            ms = _median_ms(torch, stream, lambda r: env.fce_mix(rsets[r][0], nb, rsets[r][1], nb), RMS_SETS)
            out["copy_16MiB_cold"] = {"GBps": round(2 * nb / ms / 1e6, 1), "bytes": 2 * nb,
                                      "probe": f"fce_mix read 16 MiB + write 16 MiB, {RMS_SETS} rotating sets"}
        if "gemm" in groups:
            msink = torch.empty(env.fce_mfma_sink_floats(), dtype=torch.float32, device=dev)
            iters = 2000
            ms = _median_ms(torch, stream, lambda r: env.fce_mfma(msink, iters), 1)
            out["mfma_f16_random"] = {"TFLOPs": round(env.fce_mfma_flops(iters) / ms / 1e9, 1),
                                      "probe": "fce_mfma: v_mfma_f32_32x32x16_f16 on changing random operands"}
        if "softmax" in groups:
            # vendor-written streams over the same 1 GiB buffers (beyond the MALL):
            # the runtime's device-to-device copy and memset, and torch's own fill
            sd, so = bufs["softmax"]
            nb = sd.numel() * sd.element_size()
            ms = _median_ms(torch, stream, lambda r: so.copy_(sd), 1)
            out["vendor_copy_1GiB"] = {"GBps": round(2 * nb / ms / 1e6, 1), "bytes": 2 * nb,
                                       "probe": "torch copy_ of a 1 GiB tensor (the HIP runtime's device copy)"}
            # the runtime's own memset, through the HIP runtime torch already mapped
            import ctypes
            if fc._RUNTIMES:
                hip = ctypes.CDLL(sorted(fc._RUNTIMES)[0])
                hip.hipMemsetAsync.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p]
                hip.hipMemsetAsync.restype = ctypes.c_int
                sh = ctypes.c_void_p(stream.cuda_stream)
                ms = _median_ms(torch, stream, lambda r: hip.hipMemsetAsync(so.data_ptr(), 0, nb, sh), 1)
                out["vendor_memset_1GiB"] = {"GBps": round(nb / ms / 1e6, 1), "bytes": nb,
                                             "probe": "hipMemsetAsync of a 1 GiB buffer (the HIP runtime's fill)"}
            ms = _median_ms(torch, stream, lambda r: so.fill_(1.0), 1)
            out["vendor_fill_1GiB"] = {"GBps": round(nb / ms / 1e6, 1), "bytes": nb,
                                       "probe": "torch fill_(1.0) of a 1 GiB tensor (torch's fill kernel)"}
            # the flat stream shape of this library's probes over the same buffers
            ms = _median_ms(torch, stream, lambda r: env.fce_flat(None, so, nb), 1)
            out["flat_write_1GiB"] = {"GBps": round(nb / ms / 1e6, 1), "bytes": nb,
                                      "probe": "fce_flat write: one 16-byte vector per lane, 4 KiB workgroups"}
            ms = _median_ms(torch, stream, lambda r: env.fce_flat(sd, so, nb), 1)
            out["flat_copy_1GiB"] = {"GBps": round(2 * nb / ms / 1e6, 1), "bytes": 2 * nb,
                                     "probe": "fce_flat copy: one 16-byte vector per lane, 4 KiB workgroups"}
    return out


def measure_torch_rows(torch, stream, groups, bufs):
    """The same work as PyTorch eager ops (one library kernel per operator,
    intermediates through HBM): the unfused baseline a user would otherwise
    run.  Times in us per call."""
    F = torch.nn.functional
    out = {}
    if "chain" in groups:
        sets, coef = bufs["chain"]
        a, b = coef[8]
        al, bl = [float(v) for v in a], [float(v) for v in b]

        def chain(r):
            y = sets[r][0]
            for st in range(8):
                y = y * al[st] + bl[st]
                if st % 2 == 0:
                    y = torch.relu(y)
            return y
        out["chain_K8_us"] = round(_median_ms(torch, stream, chain, CHAIN_SETS) * 1e3, 2)
    if "decode" in groups:
        dsets = bufs["decode"]
        out["decode_us"] = round(_median_ms(
            torch, stream, lambda r: F.gelu(torch.addmm(dsets[r][2], dsets[r][0], dsets[r][1])) + dsets[r][3],
            DECODE_SETS) * 1e3, 2)
        out["decode_matmul_only_us"] = round(_median_ms(
            torch, stream, lambda r: torch.matmul(dsets[r][0], dsets[r][1]), DECODE_SETS) * 1e3, 2)
    if "gemm" in groups:
        A, B, bias, R = bufs["gemm"]
        out["gemm_4096_us"] = round(_median_ms(
            torch, stream, lambda r: F.gelu(torch.addmm(bias, A, B)) + R, 1, iters=11) * 1e3, 2)
        out["gemm_4096_matmul_only_us"] = round(_median_ms(
            torch, stream, lambda r: torch.matmul(A, B), 1, iters=11) * 1e3, 2)
    if "softmax" in groups:
        sd, _ = bufs["softmax"]
        S = sd.shape[-1]
        mask = torch.ones((S, S), dtype=torch.bool, device=sd.device).triu(1)

        def sm(r):
            return torch.softmax((sd.float() * SCALE).masked_fill(mask, float("-inf")), -1).to(torch.bfloat16)
        out["softmax_us"] = round(_median_ms(torch, stream, sm, 1, iters=3) * 1e3, 2)
    if "rmsnorm" in groups:
        rsets, grms = bufs["rmsnorm"]
        out["rmsnorm_us"] = round(_median_ms(
            torch, stream,
            lambda r: rsets[r][0] * torch.rsqrt(rsets[r][0].pow(2).mean(-1, keepdim=True) + RMS_EPS) * grms,
            RMS_SETS) * 1e3, 2)
    if "attention" in groups:
        qa, ka, va, kta = bufs["attention"]
        S = qa.shape[-2]
        mask = torch.ones((S, S), dtype=torch.bool, device=qa.device).triu(1)

        def att(r):
            s = torch.matmul(qa, kta).float() * SCALE
            p = torch.softmax(s.masked_fill(mask, float("-inf")), -1).to(torch.bfloat16)
            return torch.matmul(p, va)
        out["attention_us"] = round(_median_ms(torch, stream, att, 1, iters=3) * 1e3, 2)
        # the vendor's fused attention (torch SDPA restricted to its flash
        # backend: where that backend cannot run, the call raises instead of
        # falling back to the score-materialising math path)
        try:
            from torch.nn.attention import sdpa_kernel, SDPBackend
            BH, D = qa.shape[0], qa.shape[-1]
            q4, k4, v4 = (x.view(BH // 16, 16, S, D) for x in (qa, ka, va))
            with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
                out["attention_sdpa_flash_us"] = round(_median_ms(
                    torch, stream, lambda r: F.scaled_dot_product_attention(q4, k4, v4, is_causal=True, scale=SCALE),
                    1, iters=11) * 1e3, 2)
        except Exception as ex:  # backend missing on this build: no figure
            out["attention_sdpa_flash_error"] = f"{type(ex).__name__}: {str(ex)[:120]}"
    torch.cuda.synchronize()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the timed oracle sample on the host cores (the parity checks against the "
                         "oracle before the timed steps always run)")
    ap.add_argument("--copy-calib", action="store_true",
                    help="run one plain 1 GiB device copy before the timed region (a known-size "
                         "kernel that scales the FETCH_SIZE/WRITE_SIZE counters)")
    ap.add_argument("--rows", default="chain,affine,decode,gemm,softmax,attention,rmsnorm",
                    help="comma list of row groups to run (default: all)")
    ap.add_argument("--no-references", action="store_true",
                    help="skip the stream/MFMA reference probes (libfcenv.so) timed after the steps")
    ap.add_argument("--no-model", action="store_true",
                    help="skip the cost-model calibration and validation rows (launch cost, t(n) fit, "
                         "fat sweep, all split plans, graph replay) timed after the steps")
    ap.add_argument("--no-torch-rows", action="store_true",
                    help="skip the PyTorch eager (unfused library) rows timed after the steps")
    ap.add_argument("--min-row-samples", type=int, default=MIN_ROW_SAMPLES,
                    help="event pairs per row at least: steps beyond --steps are run after the timed "
                         "region for the per-row medians (0: only the timed steps, e.g. under counters)")
    ap.add_argument("--graph", action="store_true",
                    help="time each row as one replay of a HIP graph captured from its calls")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on exactly one GPU: every kernel of the hot path works on one "
              "device's share of the data; sharding across GPUs is not implemented", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gemm_epilogues_amd as fc
    import synth

    groups = set(args.rows.split(","))
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    props = torch.cuda.get_device_properties(dev)
    log(f"device: {props.name} CUs={props.multi_processor_count} gcn={getattr(props, 'gcnArchName', '?')}")

    # ---------------------------------------------------------------- inputs (resident in HBM)
    steps = []                      # callables(timer) making up one step
    comp = {}
    bufs = {}                       # device inputs, for the reference probes and the torch rows

    if "chain" in groups:
        log("inputs: chain")
        sets = []
        for r in range(CHAIN_SETS):
            x, _, _ = synth.chain_inputs(CHAIN_N, 1, salt=r)
            xd = torch.from_numpy(x).to(dev)
            sets.append((xd, torch.empty_like(xd), torch.empty_like(xd)))
        coef = {K: synth.chain_inputs(1, K)[1:] for K in CHAIN_KS}
        sink = torch.empty(fc.fc_chain_scratch_floats(CHAIN_N, FAT_K, fc.FC_CHAIN_FAT, FAT_T),
                           dtype=torch.float32, device=dev)
        bufs["chain"] = (sets, coef)
        bufs["chain_sink"] = sink

        def chain_rows(tm, step_i):
            for K in CHAIN_KS:
                a, b = coef[K]
                tm(f"chain_fused_K{K}",
                   lambda r, a=a, b=b: fc.fc_chain(sets[r][0], sets[r][1], a, b, True,
                                                   fc.FC_CHAIN_FUSED), reps=CHAIN_SETS)
                tm(f"chain_naive_K{K}",
                   lambda r, a=a, b=b: fc.fc_chain(sets[r][0], sets[r][1], a, b, True,
                                                   fc.FC_CHAIN_NAIVE, sets[r][2]), reps=CHAIN_SETS)
            a, b = coef[8]
            tm("chain_fused_K8_warm",
               lambda r: fc.fc_chain(sets[0][0], sets[0][1], a, b, True, fc.FC_CHAIN_FUSED), reps=CHAIN_SETS)
            a, b = coef[FAT_K]
            tm(f"chain_fat_K{FAT_K}_T{FAT_T}",
               lambda r: fc.fc_chain(sets[r][0], sets[r][1], a, b, True, fc.FC_CHAIN_FAT, sink, FAT_T),
               reps=CHAIN_SETS)
        steps.append(chain_rows)

    if "affine" in groups:
        log("inputs: affine chain")
        asets = []
        for r in range(AFFINE_SETS):
            x, _, _ = synth.affine_inputs(AFFINE_N, AFFINE_K, salt=r)
            xd = torch.from_numpy(x).to(dev)
            asets.append((xd, torch.empty_like(xd), torch.empty_like(xd)))
        _, aa, ab = synth.affine_inputs(1, AFFINE_K)
        bufs["affine"] = (asets, aa, ab)

        def affine_rows(tm, step_i):
            tm("affine_fused", lambda r: fc.fc_chain(asets[r][0], asets[r][1], aa, ab, False,
                                                     fc.FC_CHAIN_FUSED), reps=AFFINE_SETS)
            tm("affine_naive", lambda r: fc.fc_chain(asets[r][0], asets[r][1], aa, ab, False,
                                                     fc.FC_CHAIN_NAIVE, asets[r][2]), reps=AFFINE_SETS)
            # warm: one 8 MiB set repeated (served from the caches)
            tm("affine_fused_warm", lambda r: fc.fc_chain(asets[0][0], asets[0][1], aa, ab, False,
                                                          fc.FC_CHAIN_FUSED), reps=AFFINE_SETS)
            tm("affine_naive_warm", lambda r: fc.fc_chain(asets[0][0], asets[0][1], aa, ab, False,
                                                          fc.FC_CHAIN_NAIVE, asets[0][2]), reps=AFFINE_SETS)
        steps.append(affine_rows)

    if "decode" in groups:
        log("inputs: decode gemm 16x4096x4096")
        M, N, K = DECODE_MNK
        dsets = []
        for r in range(DECODE_SETS):
            A, B, bias, R = synth.gemm_inputs(M, N, K, salt=r)
            tdv = [torch.from_numpy(v.view(np.int16)).to(dev).view(torch.float16) for v in (A, B, bias, R)]
            # one zero-filled workspace serves every plan of a shape
            wsb = max(fc.fc_gemm_workspace_bytes(M, N, K, p) for p in PLANS)
            dsets.append(tdv + [torch.empty((M, N), dtype=torch.float16, device=dev),
                                torch.zeros(wsb, dtype=torch.uint8, device=dev)])

        bufs["decode"] = dsets

        def decode_rows(tm, step_i):
            for plan in PLANS:
                name = "decode_plan" + "".join(map(str, plan))
                tm(name, lambda r, plan=plan: fc.fc_gemm_epilogue(*dsets[r][:5], plan, dsets[r][5]),
                   reps=DECODE_SETS)
            tm("decode_plan4_warm", lambda r: fc.fc_gemm_epilogue(*dsets[0][:5], [4], dsets[0][5]),
               reps=DECODE_SETS)
        steps.append(decode_rows)

    if "gemm" in groups:
        log("inputs: gemm 4096^3")
        M, N, K = GEMM_MNK
        A, B, bias, R = synth.gemm_inputs(M, N, K)
        td = [torch.from_numpy(v.view(np.int16)).to(dev).view(torch.float16) for v in (A, B, bias, R)]
        Y = torch.empty((M, N), dtype=torch.float16, device=dev)
        bufs["gemm"] = td
        bufs["gemm_out"] = (Y,)
        ws = torch.zeros(max(fc.fc_gemm_workspace_bytes(M, N, K, p) for p in PLANS), dtype=torch.uint8,
                         device=dev)
        bufs["gemm_out"] = (Y, ws)

        def gemm_rows(tm, step_i):
            for plan in PLANS:
                name = "gemm_plan" + "".join(map(str, plan))
                tm(name, lambda r, plan=plan: fc.fc_gemm_epilogue(td[0], td[1], td[2], td[3], Y,
                                                                  plan, ws))
        steps.append(gemm_rows)

    if "softmax" in groups:
        log("inputs: softmax [8,16,2048,2048] bf16")
        BH, S = SM_B * SM_H, SM_S
        s = synth.softmax_inputs(BH, S)
        sd = torch.from_numpy(s.view(np.int16)).to(dev).view(torch.bfloat16)
        del s
        out = torch.empty_like(sd)
        bufs["softmax"] = (sd, out)
        wsb = fc.fc_softmax_workspace_bytes(BH, S, fc.FC_SOFTMAX_UNFUSED)
        smws = torch.empty(wsb, dtype=torch.uint8, device=dev)
        bufs["softmax_ws"] = smws

        def sm_rows(tm, step_i):
            for tile in SM_TILES:
                tm(f"softmax_fused_T{tile}",
                   lambda r, tile=tile: fc.fc_causal_softmax(sd, out, SCALE, tile, fc.FC_SOFTMAX_FUSED))
            tm("softmax_mask_materialise", lambda r: fc.fc_causal_mask_materialise(smws, BH, S))
            tm("softmax_unfused",
               lambda r: fc.fc_causal_softmax(sd, out, SCALE, 64, fc.FC_SOFTMAX_UNFUSED, smws))
        steps.append(sm_rows)

    if "attention" in groups:
        log("inputs: causal attention [128,2048,128] bf16")
        Qa, Ka, Va = synth.attention_inputs(ATT_BH, ATT_S, ATT_D)
        qa, ka, va = (torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16) for x in (Qa, Ka, Va))
        del Qa, Ka, Va
        oa = torch.empty_like(qa)
        kta = ka.transpose(-1, -2).contiguous()      # batched bf16 products take contiguous operands
        sc = torch.empty((ATT_BH, ATT_S, ATT_S), dtype=torch.bfloat16, device=dev)
        pa = torch.empty_like(sc)
        bufs["attention"] = (qa, ka, va, kta)

        def att_unfused():
            torch.matmul(qa, kta, out=sc)
            fc.fc_causal_softmax(sc, pa, SCALE, 64, fc.FC_SOFTMAX_FUSED)
            torch.matmul(pa, va, out=oa)

        def att_rows(tm, step_i):
            tm("attention_fused", lambda r: fc.fc_causal_attention(qa, ka, va, oa, SCALE))
            tm("attention_scores_materialised", lambda r: att_unfused())
        steps.append(att_rows)

    if "rmsnorm" in groups:
        log("inputs: rmsnorm [1024,4096] fp32")
        rsets = []
        rg = np.random.default_rng(5)
        for r in range(RMS_SETS):
            xr = torch.from_numpy(rg.standard_normal((RMS_ROWS, RMS_D), dtype=np.float32)).to(dev)
            rsets.append((xr, torch.empty_like(xr)))
        grms = torch.from_numpy((1.0 + 0.1 * rg.standard_normal(RMS_D)).astype(np.float32)).to(dev)
        rws = torch.empty(fc.fc_rmsnorm_workspace_bytes(RMS_ROWS, RMS_D, fc.FC_RMSNORM_UNFUSED),
                          dtype=torch.uint8, device=dev)
        bufs["rmsnorm"] = (rsets, grms)
        bufs["rmsnorm_ws"] = rws

        def rms_rows(tm, step_i):
            tm("rmsnorm_fused", lambda r: fc.fc_rmsnorm(rsets[r][0], grms, rsets[r][1], RMS_EPS,
                                                        fc.FC_RMSNORM_FUSED), reps=RMS_SETS)
            tm("rmsnorm_unfused", lambda r: fc.fc_rmsnorm(rsets[r][0], grms, rsets[r][1], RMS_EPS,
                                                          fc.FC_RMSNORM_UNFUSED, rws), reps=RMS_SETS)
        steps.append(rms_rows)

    if args.copy_calib:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: 1 GiB read + 1 GiB written")
        del src, dst

    # ---------------------------------------------------------------- parity before timing
    log("parity: every row against the oracle on its resident inputs (cpu_baseline leg)")
    t0 = time.perf_counter()
    parity, parity_extra = cpu_baseline_leg_parity(torch, fc, groups, bufs)
    log(f"parity ok ({time.perf_counter() - t0:.1f}s)")

    # ---------------------------------------------------------------- warmup + timed region
    tm = Timer(torch, stream, graph=args.graph)
    log(f"warmup {args.warmup} steps")
    for w in range(args.warmup):
        for f in steps:
            f(tm, w)
    torch.cuda.synchronize()
    tm.pending.clear()
    tm.ms.clear()

    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        for f in steps:
            f(tm, i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    tm.collect()
    ms_per_step = wall / max(args.steps, 1) * 1e3
    log(f"timed region {wall:.3f}s, {ms_per_step:.3f} ms/step")
    # more samples per row after the timed region, so that every row's median
    # and minimum come from at least MIN_ROW_SAMPLES event pairs (value and
    # ms_per_step stay those of the timed steps)
    extra_steps = max(0, args.min_row_samples - args.steps)
    if extra_steps:
        log(f"sampling {extra_steps} more steps per row")
        for i in range(extra_steps):
            for f in steps:
                f(tm, args.steps + i)
        torch.cuda.synchronize()
        tm.collect()
    refs = {} if args.no_references else measure_references(torch, stream, groups, bufs, fc)
    model_rows = {} if args.no_model else measure_model_rows(torch, stream, groups, bufs, fc)
    torch_rows = {} if args.no_torch_rows else measure_torch_rows(torch, stream, groups, bufs)

    # ---------------------------------------------------------------- derived numbers
    fused_bytes = 0
    fused_ms = 0.0
    if "chain" in groups:
        for K in CHAIN_KS:
            bf = fc.fc_chain_bytes(CHAIN_N, K, fc.FC_CHAIN_FUSED)
            bn = fc.fc_chain_bytes(CHAIN_N, K, fc.FC_CHAIN_NAIVE)
            tf, tn = tm.median(f"chain_fused_K{K}"), tm.median(f"chain_naive_K{K}")
            comp[f"chain_K{K}"] = {
                "fused_us": round(tf * 1e3, 2), "naive_us": round(tn * 1e3, 2),
                "naive_over_fused": round(tn / tf, 2),
                "fused_GBps": round(bf / (tf * 1e-3) / 1e9, 1),
                "fused_frac_hbm": round(bf / (tf * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                "naive_GBps": round(bn / (tn * 1e-3) / 1e9, 1),
                "launches_naive": K, "launches_fused": 1,
                "fused_min_us": round(tm.minimum(f"chain_fused_K{K}") * 1e3, 2),
            }
            fused_bytes += bf
            fused_ms += tf
        comp["chain_K8"]["fused_warm_us"] = round(tm.median("chain_fused_K8_warm") * 1e3, 2)
        tfat = tm.median(f"chain_fat_K{FAT_K}_T{FAT_T}")
        comp[f"chain_fat_K{FAT_K}_T{FAT_T}"] = {
            "us": round(tfat * 1e3, 2),
            "fat_over_fused": round(tfat / tm.median(f"chain_fused_K{FAT_K}"), 2)}
    if "affine" in groups:
        ta, tn_ = tm.median("affine_fused"), tm.median("affine_naive")
        ba = fc.fc_chain_bytes(AFFINE_N, AFFINE_K, fc.FC_CHAIN_FUSED)
        comp["affine_K8_n1048576"] = {
            "fused_us": round(ta * 1e3, 2), "naive_us": round(tn_ * 1e3, 2),
            "naive_over_fused": round(tn_ / ta, 2),
            "fused_GBps_accounted": round(ba / (ta * 1e-3) / 1e9, 1),
            "launches_naive": AFFINE_K, "launches_fused": 1,
            "fused_warm_us": round(tm.median("affine_fused_warm") * 1e3, 2),
            "naive_warm_us": round(tm.median("affine_naive_warm") * 1e3, 2),
            "fused_min_us": round(tm.minimum("affine_fused") * 1e3, 2),
            **parity_extra.get("affine", {}),
            "note": "8 MiB footprint: latency/launch-bound; cold rotation over 40 buffer sets, warm = one set "
                    "repeated; closed-form error against h*A^8 + B(A^8-1)/(A-1) with the fp32 constants"}
    if "decode" in groups:
        M, N, K = DECODE_MNK
        for plan in PLANS:
            name = "decode_plan" + "".join(map(str, plan))
            t_ = tm.median(name)
            b = fc.fc_plan_bytes(M, N, K, plan)
            comp[name] = {"us": round(t_ * 1e3, 2), "bytes": b, "GBps": round(b / (t_ * 1e-3) / 1e9, 1),
                          "frac_hbm": round(b / (t_ * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                          "launches": fc.fc_plan_launches(plan)}
        comp["decode_plan4"]["warm_us"] = round(tm.median("decode_plan4_warm") * 1e3, 2)
    if "softmax" in groups:
        BH, S = SM_B * SM_H, SM_S
        for tile in SM_TILES:
            b = fc.fc_softmax_bytes(BH, S, tile, fc.FC_SOFTMAX_FUSED)
            t = tm.median(f"softmax_fused_T{tile}")
            comp[f"softmax_fused_T{tile}"] = {
                "us": round(t * 1e3, 2), "bytes": b, "GBps": round(b / (t * 1e-3) / 1e9, 1),
                "frac_hbm": round(b / (t * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                "min_us": round(tm.minimum(f"softmax_fused_T{tile}") * 1e3, 2)}
        bu = fc.fc_softmax_bytes(BH, S, 64, fc.FC_SOFTMAX_UNFUSED)
        tu = tm.median("softmax_unfused")
        tmask = tm.median("softmax_mask_materialise")
        comp["softmax_unfused"] = {"us": round(tu * 1e3, 2), "bytes": bu,
                                   "GBps": round(bu / (tu * 1e-3) / 1e9, 1),
                                   "mask_materialise_us": round(tmask * 1e3, 2),
                                   "unfused_over_fused_T64": round(tu / tm.median("softmax_fused_T64"), 2)}
        fused_bytes += fc.fc_softmax_bytes(BH, S, 64, fc.FC_SOFTMAX_FUSED)
        fused_ms += tm.median("softmax_fused_T64")
    if "gemm" in groups:
        M, N, K = GEMM_MNK
        flops = 2 * M * N * K
        for plan in PLANS:
            name = "gemm_plan" + "".join(map(str, plan))
            t = tm.median(name)
            comp[name] = {"us": round(t * 1e3, 2), "TFLOPs": round(flops / (t * 1e-3) / 1e12, 1),
                          "frac_mfma_fp16": round(flops / (t * 1e-3) / 1e12 / FP16_PEAK_TFLOPS, 4),
                          "bytes": fc.fc_plan_bytes(M, N, K, plan), "launches": fc.fc_plan_launches(plan),
                          "min_us": round(tm.minimum(name) * 1e3, 2)}

    if "attention" in groups:
        fl = fc.fc_attention_flops(ATT_BH, ATT_S, ATT_D)
        ta, tu = tm.median("attention_fused"), tm.median("attention_scores_materialised")
        comp["attention_fused"] = {
            "us": round(ta * 1e3, 2), "TFLOPs": round(fl / (ta * 1e-3) / 1e12, 1),
            "frac_mfma_bf16": round(fl / (ta * 1e-3) / 1e12 / FP16_PEAK_TFLOPS, 4),
            "flops": fl, "bytes": fc.fc_attention_bytes(ATT_BH, ATT_S, ATT_D), "launches": 1,
            "min_us": round(tm.minimum("attention_fused") * 1e3, 2)}
        comp["attention_scores_materialised"] = {
            "us": round(tu * 1e3, 2), "over_fused": round(tu / ta, 2), "launches": 3,
            "note": "QK^T (torch bf16 matmul) -> [128,2048,2048] bf16 scores -> fc fused softmax T64 -> PV"}

    if "rmsnorm" in groups:
        bf = fc.fc_rmsnorm_bytes(RMS_ROWS, RMS_D, fc.FC_RMSNORM_FUSED)
        bu = fc.fc_rmsnorm_bytes(RMS_ROWS, RMS_D, fc.FC_RMSNORM_UNFUSED)
        tf_, tu_ = tm.median("rmsnorm_fused"), tm.median("rmsnorm_unfused")
        comp["rmsnorm_1024x4096"] = {
            "fused_us": round(tf_ * 1e3, 2), "unfused_us": round(tu_ * 1e3, 2),
            "unfused_over_fused": round(tu_ / tf_, 2),
            "fused_GBps": round(bf / (tf_ * 1e-3) / 1e9, 1),
            "fused_frac_hbm": round(bf / (tf_ * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "ledger_bytes_fused": bf, "ledger_bytes_unfused": bu, "launches_fused": 1, "launches_unfused": 4}

    value = fused_bytes / (fused_ms * 1e-3) / 1e9 if fused_ms > 0 else None

    # roofline of the dominant kernel of `value`: the fused softmax at tile 64
    roofline = None
    if "softmax" in groups:
        BH, S = SM_B * SM_H, SM_S
        b = fc.fc_softmax_bytes(BH, S, 64, fc.FC_SOFTMAX_FUSED)
        t = tm.median("softmax_fused_T64") * 1e-3
        ach = b / t / 1e9
        roofline = {"bound": "hbm", "kernel": "softmax_fused_kernel<4,bf16> tile 64",
                    "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": round(ach / HBM_PEAK_GBPS, 4),
                    "avg_launch_us": round(t * 1e6, 2), "algorithmic_bytes": b,
                    "traffic": load_traffic("softmax_fused_T64",
                                            os.path.join(ROOT, "gemm_epilogues_amd", "csrc", "softmax.hip"))}
    others = []
    if "chain" in groups:
        K = 8
        b = fc.fc_chain_bytes(CHAIN_N, K, fc.FC_CHAIN_FUSED)
        t = tm.median(f"chain_fused_K{K}") * 1e-3
        others.append({"bound": "hbm", "kernel": "chain_fused_kernel<8,relu> n=16,777,216",
                       "achieved": round(b / t / 1e9, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                       "frac": round(b / t / 1e9 / HBM_PEAK_GBPS, 4), "avg_launch_us": round(t * 1e6, 2),
                       "algorithmic_bytes": b,
                       "traffic": load_traffic("chain_fused_K8",
                                               os.path.join(ROOT, "gemm_epilogues_amd", "csrc", "chain.hip"))})
    if "gemm" in groups:
        M, N, K = GEMM_MNK
        t = tm.median("gemm_plan4") * 1e-3
        fl = 2 * M * N * K
        others.append({"bound": "mfma", "kernel": "gemm_ring_kernel<bias+gelu+res> 256x256 plan [4]",
                       "achieved": round(fl / t / 1e12, 1), "peak": FP16_PEAK_TFLOPS, "unit": "TFLOP/s",
                       "frac": round(fl / t / 1e12 / FP16_PEAK_TFLOPS, 4), "avg_launch_us": round(t * 1e6, 2),
                       "algorithmic_flops": fl,
                       "traffic": load_traffic("gemm_plan4",
                                               os.path.join(ROOT, "gemm_epilogues_amd", "csrc", "gemm.hip"))})
    if "decode" in groups:
        M, N, K = DECODE_MNK
        b = fc.fc_plan_bytes(M, N, K, [4])
        t = tm.median("decode_plan4") * 1e-3
        others.append({"bound": "hbm", "kernel": "gemm_decode_kernel<bias+gelu+res> 16x4096x4096 plan [4]",
                       "achieved": round(b / t / 1e9, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                       "frac": round(b / t / 1e9 / HBM_PEAK_GBPS, 4), "avg_launch_us": round(t * 1e6, 2),
                       "algorithmic_bytes": b,
                       "traffic": load_traffic("decode_plan4",
                                               os.path.join(ROOT, "gemm_epilogues_amd", "csrc", "gemm.hip"))})

    def attach_reference(obj, key, field):
        c = refs.get(key)
        if obj is not None and c:
            obj["reference"] = c[field]
            obj["frac_of_reference"] = round(obj["achieved"] / c[field], 4)
            obj["reference_probe"] = c["probe"]

    attach_reference(roofline, "mix_softmax_T64", "GBps")
    if roofline is not None:
        vend = {k: refs[k]["GBps"] for k in ("vendor_copy_1GiB", "vendor_memset_1GiB", "vendor_fill_1GiB",
                                             "flat_write_1GiB", "flat_copy_1GiB") if k in refs}
        if vend:
            roofline["plain_streams_1GiB_GBps"] = vend
            roofline["frac_of_fastest_plain_stream"] = round(roofline["achieved"] / max(vend.values()), 4)
    for o in others:
        if o["kernel"].startswith("chain_fused"):
            attach_reference(o, "copy_64MiB_cold", "GBps")
        elif o["kernel"].startswith("gemm_ring"):
            attach_reference(o, "mfma_f16_random", "TFLOPs")
        elif o["kernel"].startswith("gemm_decode"):
            attach_reference(o, "read_32MiB_cold", "GBps")
    if "softmax_fused_T2048" in comp and "mix_softmax_T2048" in refs:
        comp["softmax_fused_T2048"]["frac_of_reference"] = round(
            comp["softmax_fused_T2048"]["GBps"] / refs["mix_softmax_T2048"]["GBps"], 4)
    if torch_rows:
        pairs = {"chain_K8_us": ("chain_K8", "fused_us"), "decode_us": ("decode_plan4", "us"),
                 "gemm_4096_us": ("gemm_plan4", "us"), "softmax_us": ("softmax_fused_T64", "us"),
                 "attention_us": ("attention_fused", "us"), "attention_sdpa_flash_us": ("attention_fused", "us"),
                 "rmsnorm_us": ("rmsnorm_1024x4096", "fused_us")}
        for k, (row, f) in pairs.items():
            if k in torch_rows and row in comp:
                torch_rows[k.replace("_us", "_speedup_fused_vs_torch")] = round(torch_rows[k] / comp[row][f], 2)
        comp["torch_eager"] = torch_rows

    if "rmsnorm" in groups:
        b = fc.fc_rmsnorm_bytes(RMS_ROWS, RMS_D, fc.FC_RMSNORM_FUSED)
        t = tm.median("rmsnorm_fused") * 1e-3
        o = {"bound": "hbm", "kernel": "rmsnorm_fused_kernel<4> [1024,4096] fp32",
             "achieved": round(b / t / 1e9, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
             "frac": round(b / t / 1e9 / HBM_PEAK_GBPS, 4), "avg_launch_us": round(t * 1e6, 2),
             "algorithmic_bytes": b,
             "traffic": load_traffic("rmsnorm_fused", os.path.join(ROOT, "gemm_epilogues_amd", "csrc", "rmsnorm.hip"))}
        attach_reference(o, "copy_16MiB_cold", "GBps")
        others.append(o)
    if "attention" in groups:
        fl = fc.fc_attention_flops(ATT_BH, ATT_S, ATT_D)
        t = tm.median("attention_fused") * 1e-3
        o = {"bound": "mfma", "kernel": "attention_fwd_kernel [128,2048,128] bf16 causal",
             "achieved": round(fl / t / 1e12, 1), "peak": FP16_PEAK_TFLOPS, "unit": "TFLOP/s",
             "frac": round(fl / t / 1e12 / FP16_PEAK_TFLOPS, 4), "avg_launch_us": round(t * 1e6, 2),
             "algorithmic_flops": fl, "algorithmic_bytes": fc.fc_attention_bytes(ATT_BH, ATT_S, ATT_D),
             "traffic": load_traffic("attention_fused",
                                     os.path.join(ROOT, "gemm_epilogues_amd", "csrc", "attention.hip"))}
        attach_reference(o, "mfma_f16_random", "TFLOPs")
        others.append(o)

    if model_rows:
        meas = model_rows.pop("_measured", {})
        launch_s = model_rows["launch_us"] * 1e-6
        hbm = refs.get("copy_64MiB_cold", {}).get("GBps")
        mm_us = torch_rows.get("gemm_4096_matmul_only_us") if torch_rows else None
        if mm_us:
            flops_ps, p_src = 2.0 * 4096 ** 3 / (mm_us * 1e-6), "torch.matmul fp16 4096^3 (vendor GEMM) rate"
        elif "mfma_f16_random" in refs:
            flops_ps, p_src = refs["mfma_f16_random"]["TFLOPs"] * 1e12, "random-operand MFMA probe"
        else:
            flops_ps, p_src = None, None
        if hbm and flops_ps and meas:
            m = fc.cost_model(hbm * 1e9, flops_ps, launch_s, levels=((512, 1.0),), spill_factor=3.0)
            val = {"calibration": {"hbm_GBps": hbm, "hbm_source": "copy_64MiB_cold reference",
                                   "TFLOPs": round(flops_ps / 1e12, 1), "flops_source": p_src,
                                   "launch_us": model_rows["launch_us"],
                                   "register_rule": "512 live registers per lane (one wave per SIMD), x3 beyond"}}

            def validate(model):
                res = {}
                for shape, (M, N, K) in (("decode", DECODE_MNK), ("gemm", GEMM_MNK)):
                    st = fc.fc_gemm_epilogue_stages(M, N, K)
                    rows = {}
                    for (sh, plan), t in meas.items():
                        if sh != shape:
                            continue
                        pred = fc.fc_segments_time(st, list(plan), 2, model)
                        rows["".join(map(str, plan))] = {"measured_us": round(t * 1e6, 2),
                                                         "model_us": round(pred * 1e6, 2),
                                                         "model_over_measured": round(pred / t, 3)}
                    if rows:
                        best_model, _ = fc.fc_best_split(st, 2, model)
                        best_meas = min(((t, p) for (sh, p), t in meas.items() if sh == shape))[1]
                        res[shape] = {"plans": rows, "model_best": best_model, "measured_best": list(best_meas)}
                return res
            val.update(validate(m))
            # The same model with the register rule replaced by the occupancy steps the fat
            # probe measures on this device: (live registers, time / time at the fewest
            # registers) for every unspilled point, the spilled point's ratio beyond them.
            sweep = model_rows.get("fat_sweep_K4", {}).get("rows", [])
            base = next((r["us"] for r in sweep if r["T"] == 0), None)
            pts = sorted((r["vgprs"] + r["agprs"], r["us"] / base) for r in sweep
                         if base and r["scratch_bytes_per_lane"] == 0)
            spilled = [r["us"] / base for r in sweep if base and r["scratch_bytes_per_lane"] > 0]
            if pts and spilled:
                levels, fmax = [], 0.0
                for regs, f in pts:                  # strictly increasing levels, non-decreasing factors
                    fmax = max(fmax, f)
                    if not levels or regs > levels[-1][0]:
                        levels.append((regs, round(fmax, 3)))
                mo = fc.cost_model(hbm * 1e9, flops_ps, launch_s, levels=tuple(levels[:8]),
                                   spill_factor=round(max(spilled[0], fmax), 3))
                val["occupancy_rule"] = {"levels": levels[:8], "spill_factor": round(max(spilled[0], fmax), 3),
                                         "source": "fat probe sweep (K = 4): time over the T = 0 point",
                                         **validate(mo)}
            model_rows["validation"] = val
        comp["cost_model"] = model_rows

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle on host cores)")
        cpu = cpu_baseline()

    line = {
        "metric": METRIC,
        "value": round(value, 1) if value else None,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": ("fused pointwise chain n=16,777,216 fp32 K in {2,3,4,6,8} (naive, fused, fat K=4 T=48) "
                         "+ causal scaled softmax [8,16,2048,2048] bf16 (fused tiles 64/128/256/none, unfused "
                         "5-pass + mask) + GEMM+bias+GELU+residual 4096^3 and 16x4096x4096 fp16 plans "
                         "[1,1,1,1],[1,3],[2,2],[4] + affine chain n=1,048,576 K=8 + causal attention "
                         "[128,2048,128] bf16 (one kernel vs scores materialised) + RMSNorm [1024,4096] fp32 "
                         "(fused vs 4 passes)"),
            "timing": ("HIP event pair per row around " +
                       ("one replay of the row's captured HIP graph" if args.graph else "host launches") +
                       f"; per-row medians and minima over {args.steps + extra_steps} samples"),
            "value_definition": "algorithmic bytes of fused chain (K=2,3,4,6,8) + fused softmax (tile 64) / their summed kernel time",
            "gemm_TFLOPs_plan4": comp.get("gemm_plan4", {}).get("TFLOPs"),
            "device": props.name,
        },
        "roofline": roofline,
        "parity": parity,
        "rooflines_other": others,
        "references": refs,
        "cpu_baseline": cpu,
        "components": comp,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
