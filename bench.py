"""Benchmark of the Positional-LSH ALiBi attention kernel on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the GPU hot path (block intervals, multiplicities,
QK^T, weighted online softmax, PV, normalisation: one library call) over one
batch of seeded synthetic inputs already resident in HBM, with the hash
tables (drawn and built on the host once, timed separately) resident too.
Before the W warmup steps the same call runs untimed for --settle-s seconds:
the GPU's clock ramps up over the first ~0.1 s of load, and the timed steps
measure the steady state.
Prints ONE JSON line on stdout; progress goes to stderr.

    python bench.py --copy-calibration MIB

runs a plain device-to-device copy of MIB MiB a few times instead (the known
byte count against which the HBM byte counters are scaled) and prints one
JSON line describing it.

    python bench.py --sweep

times every workload (tiny fp32 through n = 524288) and prints one JSON line
per workload, with the estimate's error against exact ALiBi.

    python bench.py --crossover

times the estimator (one library call) against the dense exact-ALiBi kernel
(plsh_exact_alibi_attention) on the Mistral-shaped workload for a range of
sequence lengths and prints one JSON line per length.

The default run also times, outside the timed steps and on the same inputs,
the exact-ALiBi kernel ("exact_alibi_comparator"), fixed blocks through the
estimator ("fixed_blocks_baseline"), the unfused per-sample form
("unfused_ablation"), the per-sample walk inside one kernel
("walk_ablation") and the backward for fixed tables ("backward", with the
variant that starts from a saved forward's output and row statistics);
--no-comparators skips them (profiling runs).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np
import torch

from approximate_long_context_amd import plsh, workloads as W

HERE = os.path.dirname(os.path.abspath(__file__))
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
# the measured forward kernel's source (its hash keys the committed counter runs)
KERNEL_SRCS = [os.path.join(HERE, "approximate_long_context_amd", "csrc", f)
               for f in ("plsh_fwd.hip", "plsh_fwd.h", "plsh_device.h")]
FLUSH_BYTES = 1 << 30          # > the 256 MB Infinity Cache and every L2
TRAFFIC_FILE = os.path.join(HERE, "profiles", "traffic.json")
MFMA_FILE = os.path.join(HERE, "profiles", "mfma.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def copy_calibration(mib: int) -> None:
    """A plain copy kernel of known size, for scaling FETCH_SIZE / WRITE_SIZE."""
    dev = torch.device("cuda:0")
    nbytes = mib << 20
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    reps = 5
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": True, "bytes_read_per_copy": nbytes,
                      "bytes_written_per_copy": nbytes, "copies": reps}), flush=True)


def error_stats(est: torch.Tensor, ref: torch.Tensor) -> dict:
    """max |est - ref|, ||est - ref||_F / ||ref||_F, and the per-row
    infinity norm ||est_i - ref_i||_inf / ||ref_i||_inf (median and max over
    rows), over the whole output (fp32 on the device)."""
    e, r = est.float(), ref.float()
    d = e - r
    row_err = d.abs().amax(dim=-1)
    row_ref = r.abs().amax(dim=-1).clamp_min(torch.finfo(torch.float32).tiny)
    rel_rows = (row_err / row_ref).flatten()
    return {"rows": "all", "max_abs": float(d.abs().max()),
            "rel_fro": float(d.norm() / r.norm()),
            "row_inf_rel_median": float(rel_rows.median()), "row_inf_rel_max": float(rel_rows.max())}


def exact_reference(w: W.Workload, qd, kd, vd) -> torch.Tensor:
    """Exact ALiBi on the device: the dense exact-ALiBi kernel (bf16; checked
    against the oracle's exact ALiBi in the GPU tests)."""
    return plsh.exact_alibi_attention(qd, kd, vd, w.sigma, causal=w.causal)


def dense_flops(w: W.Workload) -> float:
    """QK^T and PV flops of exact attention: 4 d per (row, key) pair."""
    pairs = w.n * (w.n + 1) / 2 if w.causal else float(w.n) * w.n
    return 4.0 * w.d * w.batch * w.heads * pairs


def sdpa_flash_ms(qd, kd, vd, causal: bool, reps: int):
    """torch's scaled_dot_product_attention restricted to its flash backend
    (no bias: a lower bound on what dense exact attention can cost on this
    stack), GQA by enable_gqa; ms per call, or the reason it is unavailable.
    The backend is forced so that no other path (the math path's batched
    products in particular) runs instead."""
    import torch.nn.functional as F
    from torch.nn.attention import SDPBackend, sdpa_kernel
    try:
        with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
            fn = lambda: F.scaled_dot_product_attention(qd, kd, vd, is_causal=causal,
                                                        enable_gqa=qd.shape[1] != kd.shape[1])
            fn()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / reps, None
    except RuntimeError as ex:
        return None, str(ex)[:200]


def time_calls(fn, reps: int, launches_per_call: int = 1):
    """(ms per call by events around the calls, ms per attention kernel by the
    library's kernel timer)."""
    dev = torch.device("cuda:0")
    fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    plsh.kernel_timer(True)
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    launches, total = plsh.kernel_timer_read()
    plsh.kernel_timer(False)
    assert launches == reps * launches_per_call, (launches, reps, launches_per_call)
    return e0.elapsed_time(e1) / reps, total / launches


def graph_calls_ms(fn, reps: int) -> float:
    """ms per call when one call, captured once in a HIP graph, is replayed
    `reps` times back to back: the device's time per call without the host's
    per-call work in the binding (fn must pass its output and workspace, so
    the captured call neither allocates nor fills memory)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del g
    return ms


def crossover() -> None:
    """Estimator vs exact ALiBi over n on the Mistral-shaped workload."""
    import dataclasses
    dev = torch.device("cuda:0")
    base = W.get("mistral-7b-n16384-s20")
    for n in (1024, 2048, 4096, 8192, 16384, 32768, 65536):
        w = dataclasses.replace(base, n=n, name=f"mistral-shape-n{n}-s{base.s}")
        q, k, v = W.make_qkv(w)
        qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
        dt = plsh.sample_tables(w.hash_seed, n, w.sigma, w.s).to(dev)
        out = torch.empty_like(qd)
        t0 = time.perf_counter()   # let the clock settle (as in the main run)
        while time.perf_counter() - t0 < 0.5:
            for _ in range(10):
                plsh.attention(qd, kd, vd, w.sigma, w.s, dt, causal=w.causal, out=out)
            torch.cuda.synchronize()
        reps_lsh = 50
        reps_exact = max(2, min(20, int(2e8 // (n * n))))
        lsh_ms, lsh_kernel_ms = time_calls(
            lambda: plsh.attention(qd, kd, vd, w.sigma, w.s, dt, causal=w.causal, out=out), reps_lsh)
        ex_ms, ex_kernel_ms = time_calls(
            lambda: plsh.exact_alibi_attention(qd, kd, vd, w.sigma, causal=w.causal, out=out), reps_exact)
        fa_ms, _ = sdpa_flash_ms(qd, kd, vd, w.causal, reps_exact)
        rec = {"crossover": True, "workload": w.name, "n": n, "lsh_call_ms": lsh_ms,
               "lsh_attention_kernel_ms": lsh_kernel_ms, "exact_ms": ex_ms,
               "exact_tflops": dense_flops(w) / (ex_kernel_ms / 1e3) / 1e12,
               "exact_over_lsh": ex_ms / lsh_ms,
               "torch_sdpa_flash_no_bias_ms": fa_ms,
               "torch_sdpa_flash_tflops": None if fa_ms is None else dense_flops(w) / (fa_ms / 1e3) / 1e12}
        log(f"[crossover] n={n}: estimator {lsh_ms:.3f} ms, exact {ex_ms:.3f} ms "
            f"({rec['exact_tflops']:.0f} TFLOP/s), ratio {rec['exact_over_lsh']:.2f}")
        print(json.dumps(rec), flush=True)
        del qd, kd, vd, out, dt
        torch.cuda.empty_cache()


SWEEP = ["tiny-f32-n512", "slopes-n4096", "qwen3-0.6b-n8192-s10", "qwen3-0.6b-n8192-s20",
         "mistral-7b-n16384-s10", "mistral-7b-n16384-s20", "mistral-7b-n16384-s40",
         "long-n65536", "long-n131072", "long-n524288"]


def sweep(settle_s: float) -> None:
    """Every workload: the call's time and throughput, the attention kernel's
    time and HBM roofline fraction, (informational) the estimate's error
    against exact ALiBi on the whole output, the exact output from the dense
    exact-ALiBi kernel, and the time of the backward from a saved forward
    (bf16 workloads; the fp32 one has neither an exact nor a backward
    kernel).  One JSON line per workload."""
    dev = torch.device("cuda:0")
    for name in SWEEP:
        w = W.get(name)
        q, k, v = W.make_qkv(w)
        tables = plsh.sample_tables(w.hash_seed, w.n, w.sigma, w.s)
        pairs_alg, pairs_distinct = plsh.count_work(tables, w.causal)
        dt = tables.to(dev)
        qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
        out = torch.empty_like(qd)
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < settle_s:
            for _ in range(10):
                plsh.attention(qd, kd, vd, w.sigma, w.s, dt, causal=w.causal, out=out)
            torch.cuda.synchronize()
        reps = 50 if w.n <= 16384 else 10
        ms, kernel_ms = time_calls(lambda: plsh.attention(qd, kd, vd, w.sigma, w.s, dt, causal=w.causal,
                                                          out=out), reps)
        warm = per_call_stats(lambda: plsh.attention(qd, kd, vd, w.sigma, w.s, dt, causal=w.causal, out=out),
                              reps)
        wsd = torch.empty(max(1, plsh.workspace_size(w.n, w.heads, w.s, qd.dtype)), dtype=torch.uint8, device=dev)
        graph_ms = graph_calls_ms(lambda: plsh.attention(qd, kd, vd, w.sigma, w.s, dt, causal=w.causal, out=out,
                                                         workspace=wsd), reps)
        del wsd
        B, H, Hkv, n, d, s = w.batch, w.heads, w.kv_heads, w.n, w.d, w.s
        bytes_min = w.esz * B * n * d * (2 * H + 2 * Hkv)
        err = error_stats(out, exact_reference(w, qd, kd, vd)) if w.dtype == "bf16" else None
        bwd = None
        if w.dtype == "bf16" and s <= 124:
            # the backward from a saved forward (output and row statistics)
            g = torch.Generator().manual_seed(3)
            dod = torch.randn(q.shape, generator=g).to(q.dtype).to(dev)
            o_s, l_s = plsh.attention_with_lse(qd, kd, vd, w.sigma, w.s, dt, causal=w.causal)
            bw_ms, _ = time_calls(lambda: plsh.attention_backward(qd, kd, vd, dod, w.sigma, w.s, dt,
                                                                  causal=w.causal, out=o_s, lse2=l_s),
                                  5 if n <= 16384 else 3, 2)
            bwd = {"saved_forward_backward_ms": bw_ms, "over_forward_call": bw_ms / ms}
            del dod, o_s, l_s
        del qd, kd, vd, out
        torch.cuda.empty_cache()
        rec = {"sweep": True, "workload": name, "batch": B, "heads": H, "kv_heads": Hkv, "n": n, "d": d,
               "s": s, "causal": w.causal, "dtype": w.dtype, "ms_per_call": ms, "kernel": kernel_name(w),
               "kernel_ms": kernel_ms, "rows_samples_per_s": B * H * n * s / (ms / 1e3),
               "useful_tflops": 4.0 * d * B * pairs_distinct / (ms / 1e3) / 1e12,
               "s_walk_equivalent_tflops": 4.0 * d * B * pairs_alg / (ms / 1e3) / 1e12,
               "hbm_frac_kernel": bytes_min / (kernel_ms / 1e3) / 1e9 / PEAK_HBM_GBS,
               "roofline": roofline_entry(w, pairs_distinct, kernel_ms, ms), "warm": warm,
               "graph_replay_ms_per_call": graph_ms,
               "error_vs_exact_alibi": err, "backward": bwd, "kernel_sha": kernel_sha()}
        log(f"[sweep] {name}: {ms:.4f} ms/call, kernel {kernel_ms:.4f} ms, "
            f"{rec['rows_samples_per_s']:.3g} rows*samples/s, HBM frac {rec['hbm_frac_kernel']:.2f}, "
            f"rel. error vs exact {'n/a' if err is None else format(err['rel_fro'], '.3f')}, "
            f"backward {'n/a' if bwd is None else format(bwd['saved_forward_backward_ms'], '.3f') + ' ms'}")
        print(json.dumps(rec), flush=True)
        del q, k, v


def issued_pairs(t: plsh.Tables, causal: bool) -> int:
    """(row, key) pairs the MFMA kernel evaluates per batch element: each 32-row
    wave computes the 32-key tiles of its group's key range, from the
    smallest block start of the group's rows (rounded down to 32) to the
    group's end (causal) or its largest block end (rounded up to 32)."""
    n, total = t.n, 0
    x = np.arange(n)
    for h in range(t.heads):
        lo = np.full(n, n)
        hi = np.zeros(n, dtype=np.int64)
        for k in range(t.s):
            st = t.starts_of(h, k).astype(np.int64)
            idx = np.searchsorted(st, x, side="right") - 1
            lo = np.minimum(lo, st[idx])
            hi = np.maximum(hi, st[idx + 1])
        for r0 in range(0, n, 32):
            u0 = (int(lo[r0:r0 + 32].min()) // 32) * 32
            u1 = r0 + 32 if causal else ((int(hi[r0:r0 + 32].max()) + 31) // 32) * 32
            total += (u1 - u0) * 32
    return total


def measured_mfma(workload: str):
    """bf16 MFMA flops per launch from the committed counter run
    (SQ_INSTS_VALU_MFMA_MOPS_BF16, 512 flops per unit), if taken on the
    current kernel source; else None."""
    try:
        ent = json.load(open(MFMA_FILE)).get(workload)
    except (OSError, ValueError):
        return None
    if not ent or ent.get("kernel_sha") != kernel_sha():
        return None
    return ent.get("bf16_flops_per_launch")


def kernel_sha() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SRCS:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def kernel_name(w: W.Workload) -> str:
    """The attention kernel the library dispatches for this workload."""
    if w.dtype == "bf16" and w.s <= 255:
        return f"attn_fwd_kernel<{w.d}, {'true' if w.causal else 'false'}>"
    return f"attn_valu_kernel<{'uint16_t' if w.dtype == 'bf16' else 'float'}, {w.d}>"


def per_call_stats(fn, reps: int, flush: torch.Tensor = None) -> dict:
    """Median and min over `reps` single calls, each synchronised: the call
    (events around it on the current stream) and its attention kernel (events
    stamped by the kernel's dispatch).  With `flush`, every call is preceded
    by a write of that buffer (>= 1 GiB: evicts the Infinity Cache and the
    L2s), so the call starts cold."""
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    calls, kerns = [], []
    for i in range(reps):
        if flush is not None:
            flush.fill_(i & 0xFF)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        plsh.kernel_timer(True)
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        launches, total = plsh.kernel_timer_read()
        plsh.kernel_timer(False)
        calls.append(e0.elapsed_time(e1))
        kerns.append(total / max(launches, 1))
    return {"reps": reps, "cold": flush is not None,
            "call_ms_median": float(np.median(calls)), "call_ms_min": float(np.min(calls)),
            "kernel_ms_median": float(np.median(kerns)), "kernel_ms_min": float(np.min(kerns))}


def roofline_entry(w: W.Workload, pairs_distinct: int, kernel_ms: float, call_ms: float) -> dict:
    """HBM roofline of the attention kernel on the algorithmic bytes, and the
    useful-FLOP rate against the bf16 peak and against this workload's own
    attainable rate min(P_bf16, AI x BW_HBM)."""
    B, H, Hkv, n, d = w.batch, w.heads, w.kv_heads, w.n, w.d
    bytes_min = w.esz * B * n * d * (2 * H + 2 * Hkv)
    f_distinct = 4.0 * d * B * pairs_distinct
    ai = f_distinct / bytes_min
    attainable = min(PEAK_BF16_TFLOPS, ai * PEAK_HBM_GBS / 1e3)
    useful_kernel = f_distinct / (kernel_ms / 1e3) / 1e12
    ach = bytes_min / (kernel_ms / 1e3) / 1e9
    return {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": ach / PEAK_HBM_GBS,
            "kernel_ms": kernel_ms, "call_ms": call_ms, "algorithmic_bytes_per_launch": bytes_min,
            "arith_intensity_flop_per_byte": ai,
            "attainable_useful_tflops": attainable,
            "attainable_pct_bf16_peak": 100.0 * attainable / PEAK_BF16_TFLOPS,
            "useful_tflops_in_kernel": useful_kernel,
            "useful_pct_bf16_peak_in_kernel": 100.0 * useful_kernel / PEAK_BF16_TFLOPS,
            "useful_tflops_per_call": f_distinct / (call_ms / 1e3) / 1e12,
            "useful_pct_bf16_peak_per_call": 100.0 * f_distinct / (call_ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS}


def companion(name: str, settle_s: float, reps: int = 50) -> dict:
    """Time, throughput and roofline of another configuration of the same
    shape (e.g. s = 40, where the useful-FLOP target lies under the HBM roof)."""
    dev = torch.device("cuda:0")
    w = W.get(name)
    q, k, v = W.make_qkv(w)
    tables = plsh.sample_tables(w.hash_seed, w.n, w.sigma, w.s)
    _, pairs_distinct = plsh.count_work(tables, w.causal)
    dt = tables.to(dev)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    out = torch.empty_like(qd)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < settle_s:
        for _ in range(10):
            plsh.attention(qd, kd, vd, w.sigma, w.s, dt, causal=w.causal, out=out)
        torch.cuda.synchronize()
    ms, kernel_ms = time_calls(lambda: plsh.attention(qd, kd, vd, w.sigma, w.s, dt, causal=w.causal, out=out),
                               reps)
    warm = per_call_stats(lambda: plsh.attention(qd, kd, vd, w.sigma, w.s, dt, causal=w.causal, out=out), reps)
    rec = {"workload": name, "s": w.s, "ms_per_call": ms, "kernel_ms": kernel_ms,
           "rows_samples_per_s": w.batch * w.heads * w.n * w.s / (ms / 1e3),
           "roofline": roofline_entry(w, pairs_distinct, kernel_ms, ms), "warm": warm}
    del qd, kd, vd, out, dt
    torch.cuda.empty_cache()
    return rec


def measured_traffic(workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel source; else None."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    ent = rec.get(workload)
    if not ent or ent.get("kernel_sha") != kernel_sha():
        return None
    return ent.get("bytes_per_launch")


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def bf16_excess(gpu: np.ndarray, ref: np.ndarray) -> float:
    """max(|gpu - ref| - half an ulp of bf16 at |ref|): the error beyond the
    rounding of the estimate itself to bf16."""
    a = np.abs(ref)
    half = np.where(a > 0, 2.0 ** (np.floor(np.log2(np.where(a > 0, a, 1.0))) - 8), 0.0)
    return float((np.abs(gpu - ref) - half).max())


def cpu_baseline(w: W.Workload, q, k, v, t, budget_s: float, gpu_out: torch.Tensor):
    """The fp64 CPU oracle as it stands, beside the GPU:
    * its LSH estimate (O3) on whole heads of the same workload, heaviest
      first, until `budget_s` seconds of CPU work (all BLAS threads): the
      reported rate; and its agreement with the GPU's output on those heads
      (max-abs, and the excess over bf16 rounding of the estimate);
    * its exact ALiBi (O1) on sampled rows of the same workload;
    * single-thread O3 on the tiny fp32 workload and on two heads of the
      per-head-slopes workload; the tiny workload also on the GPU, with the
      fp32 path's normwise and elementwise relative errors;
    * the bias-matrix errors ||L* - M~|| (max, spectral, Frobenius; O4) of
      the hashes of the workloads with n <= 4096.
    Nothing here is inside the GPU's timed steps."""
    import oracle as orc
    from threadpoolctl import threadpool_info, threadpool_limits
    dev = torch.device("cuda:0")
    qf, kf, vf = W.to_f64(q), W.to_f64(k), W.to_f64(v)
    off, st = orc.tables_from_params(w.n, t.params)
    tabs = orc.starts_per_head(off, st, w.heads, w.s)
    done_rows = 0
    heads_done = []
    results = []
    el = 0.0
    for h in range(w.heads - 1, -1, -1):   # heaviest heads first, like the GPU schedule
        g = h // (w.heads // w.kv_heads)
        t0 = time.perf_counter()
        results.append(orc.lsh_estimate(qf[:1, h:h + 1], kf[:1, g:g + 1], vf[:1, g:g + 1], [tabs[h]], w.causal))
        el += time.perf_counter() - t0
        done_rows += w.n
        heads_done.append(h)
        if el >= budget_s:
            break
    gpu64 = W.to_f64(gpu_out)
    parity_abs = max(float(np.abs(gpu64[:1, h:h + 1] - r).max()) for h, r in zip(heads_done, results))
    parity_ex = max(bf16_excess(gpu64[:1, h:h + 1], r) for h, r in zip(heads_done, results))
    threads = max([x.get("num_threads", 1) for x in threadpool_info()] + [1])

    # O1, exact ALiBi, on sampled rows of every head (all threads)
    rows = W.sample_rows(w.n, 64, seed=11)
    t0 = time.perf_counter()
    orc.exact_alibi(qf[:1], kf[:1], vf[:1], w.sigma, w.causal, rows=rows)
    ex_s = time.perf_counter() - t0
    exact_rec = {"value": len(rows) * w.heads / ex_s, "unit": "query-rows/s", "cores": threads,
                 "sample": f"fp64 oracle exact ALiBi, {len(rows)} sampled rows x {w.heads} heads "
                           f"(batch 0), {ex_s:.1f} s"}

    # single thread: the tiny fp32 workload (whole) and two heads of the
    # per-head-slopes workload
    single = {}
    w1 = W.get("tiny-f32-n512")
    q1, k1, v1 = W.make_qkv(w1)
    t1 = plsh.sample_tables(w1.hash_seed, w1.n, w1.sigma, w1.s)
    o1, s1 = orc.tables_from_params(w1.n, t1.params)
    tabs1 = orc.starts_per_head(o1, s1, w1.heads, w1.s)
    with threadpool_limits(1):
        t0 = time.perf_counter()
        ref1 = orc.lsh_estimate(W.to_f64(q1), W.to_f64(k1), W.to_f64(v1), tabs1, w1.causal)
        e1 = time.perf_counter() - t0
    single[w1.name] = {"value": w1.batch * w1.heads * w1.n * w1.s / e1, "unit": "query-rows*samples/s",
                       "cores": 1, "sample": f"whole workload, {e1 * 1e3:.1f} ms"}
    g1 = plsh.attention(q1.to(dev), k1.to(dev), v1.to(dev), w1.sigma, w1.s, t1.to(dev), causal=w1.causal)
    torch.cuda.synchronize()
    g1 = W.to_f64(g1)
    big = np.abs(ref1) >= 1e-3 * np.abs(ref1).max()
    rel = np.abs(g1 - ref1)[big] / np.abs(ref1)[big]
    fp32_rec = {"workload": w1.name, "normwise_rel": float(np.abs(g1 - ref1).max() / np.abs(ref1).max()),
                "elementwise_rel_max": float(rel.max()), "elementwise_rel_median": float(np.median(rel)),
                "elementwise_over": "entries with |ref| >= 1e-3 max|ref|"}
    w2 = W.get("slopes-n4096")
    q2, k2, v2 = W.make_qkv(w2)
    t2 = plsh.sample_tables(w2.hash_seed, w2.n, w2.sigma, w2.s)
    o2, s2 = orc.tables_from_params(w2.n, t2.params)
    tabs2 = orc.starts_per_head(o2, s2, w2.heads, w2.s)
    with threadpool_limits(1):
        t0 = time.perf_counter()
        orc.lsh_estimate(W.to_f64(q2[:1, :2]), W.to_f64(k2[:1, :2]), W.to_f64(v2[:1, :2]), tabs2[:2], w2.causal)
        e2 = time.perf_counter() - t0
    single[w2.name] = {"value": 2 * w2.n * w2.s / e2, "unit": "query-rows*samples/s", "cores": 1,
                       "sample": f"heads 0 and 1 of batch 0 (sigma 2 and 4), {e2 * 1e3:.1f} ms"}

    # O4: ||L* - M~|| of the hashes, for the workloads with n <= 4096
    matrix = {}
    for wx, tabx, heads in ((w1, tabs1, (0,)), (w2, tabs2, (0, w2.heads - 1))):
        for h in heads:
            Ls = orc.alibi_matrix(wx.n, wx.sigma[h])
            e = orc.matrix_errors(Ls, orc.mask_mean(wx.n, tabx[h]))
            matrix[f"{wx.name} head {h} (sigma {wx.sigma[h]:g}, s {wx.s})"] = e
    return {"value": done_rows * w.s / el, "unit": "query-rows*samples/s", "cores": threads,
            "kind": "oracle",
            "sample": f"fp64 oracle LSH estimate, full rows of {len(heads_done)} of {w.heads} heads "
                      f"(batch 0, heads {heads_done[0]}..{heads_done[-1]}), {done_rows} rows x s={w.s}, "
                      f"{el:.1f} s",
            "cpu_model": cpu_model(), "os_cpu_count": os.cpu_count(),
            "parity_with_gpu_max_abs": parity_abs,
            "parity_with_gpu_excess_over_bf16_rounding": parity_ex,
            "exact_alibi_oracle": exact_rec,
            "single_thread": single,
            "fp32_path_parity": fp32_rec,
            "matrix_errors": matrix}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle-s", type=float, default=1.0,
                    help="seconds of untimed calls before the warmup steps (the GPU clock ramps up "
                         "over the first ~0.1 s of load)")
    ap.add_argument("--workload", default="mistral-7b-n16384-s20")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--error-rows", type=int, default=16,
                    help="accepted for older command lines; the error against exact ALiBi is "
                         "measured on the whole output")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB")
    ap.add_argument("--crossover", action="store_true")
    ap.add_argument("--sweep", action="store_true",
                    help="every workload: time, throughput, roofline fraction, error (one line each)")
    ap.add_argument("--no-comparators", action="store_true",
                    help="skip the exact-ALiBi, fixed-blocks and unfused comparisons (profiling runs)")
    ap.add_argument("--no-percall", action="store_true",
                    help="skip the single-call warm and cold medians (profiling runs)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on exactly one GPU; --gpus above 1 is not supported "
              "(the path would shard by (batch, kv-head group) with no communication).",
              file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a HIP device"
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.crossover:
        crossover()
        return
    if args.sweep:
        sweep(min(args.settle_s, 0.5))
        return
    dev = torch.device("cuda:0")
    w = W.get(args.workload)
    log(f"[bench] workload {w.name}: {w.describe()}")

    q, k, v = W.make_qkv(w)
    t0 = time.perf_counter()
    tables = plsh.sample_tables(w.hash_seed, w.n, w.sigma, w.s)
    host_sample_ms = (time.perf_counter() - t0) * 1e3
    pairs_alg, pairs_distinct = plsh.count_work(tables, w.causal)
    dt = tables.to(dev)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    out = torch.empty_like(qd)
    torch.cuda.synchronize()

    settle_calls = 0
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < args.settle_s:
        for _ in range(20):
            plsh.attention(qd, kd, vd, w.sigma, w.s, dt, causal=w.causal, out=out)
        settle_calls += 20
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        plsh.attention(qd, kd, vd, w.sigma, w.s, dt, causal=w.causal, out=out)
    torch.cuda.synchronize()
    log(f"[bench] settled ({settle_calls} calls, {args.settle_s} s), warmup done ({args.warmup})")
    stream = torch.cuda.current_stream(dev)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    plsh.kernel_timer(True)   # HIP events stamped by the attention kernel's dispatch, every call
    e0.record(stream)
    for _ in range(args.steps):
        plsh.attention(qd, kd, vd, w.sigma, w.s, dt, causal=w.causal, out=out)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    launches, kernel_ms_total = plsh.kernel_timer_read()
    plsh.kernel_timer(False)
    assert launches == args.steps, (launches, args.steps)
    kernel_ms = kernel_ms_total / launches
    log(f"[bench] timed {args.steps} steps: {ms:.4f} ms/step, attention kernel {kernel_ms:.4f} ms")
    # single synchronised calls: warm, and cold (a 1 GiB write before each)
    one = lambda: plsh.attention(qd, kd, vd, w.sigma, w.s, dt, causal=w.causal, out=out)
    warm = cold = None
    graph_ms = rec_ms = None
    if not args.no_percall:
        warm = per_call_stats(one, 50)
        flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
        cold = per_call_stats(one, 50, flush)
        del flush
        torch.cuda.empty_cache()
        # the same call captured once in a HIP graph and replayed back to back
        wsd = torch.empty(plsh.workspace_size(w.n, w.heads, w.s, qd.dtype), dtype=torch.uint8, device=dev)
        graph_ms = graph_calls_ms(lambda: plsh.attention(qd, kd, vd, w.sigma, w.s, dt, causal=w.causal,
                                                         out=out, workspace=wsd), args.steps)
        log(f"[bench] graph-replayed calls: {graph_ms:.4f} ms per call")
        # fixed tables: the records built once, then the attention kernel
        # alone per call (an inference loop whose hashes do not change)
        if w.dtype == "bf16":
            plsh.build_records(dt, w.causal, wsd)
            rec_ms, _ = time_calls(lambda: plsh.attention_from_records(qd, kd, vd, w.sigma, w.s, dt, wsd,
                                                                       causal=w.causal, out=out), args.steps)
            log(f"[bench] records built once: {rec_ms:.4f} ms per call")
        del wsd
    if warm:
        log(f"[bench] single calls, median/min: warm {warm['call_ms_median']:.4f}/{warm['call_ms_min']:.4f} ms "
            f"(kernel {warm['kernel_ms_median']:.4f}/{warm['kernel_ms_min']:.4f}), cold "
            f"{cold['call_ms_median']:.4f}/{cold['call_ms_min']:.4f} ms (kernel {cold['kernel_ms_median']:.4f}/"
            f"{cold['kernel_ms_min']:.4f})")

    B, H, Hkv, n, d, s = w.batch, w.heads, w.kv_heads, w.n, w.d, w.s
    sec = ms / 1e3
    if not args.no_comparators:
        # the forward that also writes each row's normaliser (for a backward
        # from a saved forward), timed right after the timed steps so that
        # both run in the same state of the GPU
        o_s = torch.empty_like(qd)
        l_s = torch.empty((B, H, (n + 31) // 32 * 32), dtype=torch.float32, device=dev)
        fl_ms, fl_kernel_ms = time_calls(lambda: plsh.attention_with_lse(
            qd, kd, vd, w.sigma, w.s, dt, causal=w.causal, out=o_s, lse2=l_s), 50)
    rows_samples = B * H * n * s / sec
    f_distinct = 4.0 * d * B * pairs_distinct
    f_alg = 4.0 * d * B * pairs_alg
    bytes_min = w.esz * B * n * d * (2 * H + 2 * Hkv)
    ach_gbs = bytes_min / (kernel_ms / 1e3) / 1e9  # the attention kernel alone
    useful_tflops = f_distinct / sec / 1e12
    traffic = measured_traffic(w.name)
    issued = B * issued_pairs(tables, w.causal)
    mfma_flops = measured_mfma(w.name)

    # error of the estimate against exact ALiBi on the whole output
    # (informational): the exact output from the dense exact-ALiBi kernel,
    # which the GPU tests check against the oracle's exact ALiBi
    exact = exact_reference(w, qd, kd, vd) if w.dtype == "bf16" else None
    err = error_stats(out, exact) if exact is not None else None
    if err:
        log(f"[bench] error vs exact ALiBi: max-abs {err['max_abs']:.3e}, rel. Frobenius {err['rel_fro']:.3f}")

    # the dense exact-ALiBi kernel's time on the same inputs (informational,
    # after the timed steps)
    exact_rec = None
    if not args.no_comparators and exact is not None:
        ex_out = torch.empty_like(qd)
        ex_call = lambda: plsh.exact_alibi_attention(qd, kd, vd, w.sigma, causal=w.causal, out=ex_out)
        t_ex = time.perf_counter()  # its own load first: the clock settles for it
        while time.perf_counter() - t_ex < min(args.settle_s, 0.3):
            ex_call()
            torch.cuda.synchronize()
        ex_ms, ex_kernel_ms = time_calls(ex_call, 10)
        ex_tflops = dense_flops(w) / (ex_kernel_ms / 1e3) / 1e12
        fa_ms, fa_why = sdpa_flash_ms(qd, kd, vd, w.causal, 3)
        exact_rec = {"kernel": "exact_fwd_kernel", "ms": ex_ms, "kernel_ms": ex_kernel_ms,
                     "dense_tflop": dense_flops(w) / 1e12, "tflops": ex_tflops,
                     "pct_bf16_peak": 100.0 * ex_tflops / PEAK_BF16_TFLOPS,
                     "exact_over_lsh_call": ex_ms / ms,
                     "torch_sdpa_flash_no_bias": None if fa_ms is None else {
                         "ms": fa_ms, "tflops": dense_flops(w) / (fa_ms / 1e3) / 1e12,
                         "over_lsh_call": fa_ms / ms, "over_exact_alibi": fa_ms / ex_ms},
                     "torch_sdpa_flash_unavailable": fa_why}
        log(f"[bench] exact ALiBi kernel {ex_ms:.3f} ms ({ex_tflops:.0f} TFLOP/s), "
            f"{ex_ms / ms:.1f}x the estimator's call; torch SDPA flash (no bias) "
            f"{'unavailable' if fa_ms is None else format(fa_ms, '.3f') + ' ms'}")
        del ex_out

    # the "fixed blocks" baseline (one deterministic hash per head, pitch
    # 2 sigma = the mean random pitch, offset 0) through the same kernel:
    # its error against exact ALiBi on the whole output, and its time
    fixed_rec = None
    if not args.no_comparators and exact is not None:
        ft = plsh.fixed_block_tables(n, [2.0 * x for x in w.sigma], 1).to(dev)
        fx_out = torch.empty_like(qd)
        fx_ms, _ = time_calls(lambda: plsh.attention(qd, kd, vd, w.sigma, 1, ft, causal=w.causal, out=fx_out), 5)
        fixed_rec = {"table": "pitch 2 sigma_h, offset 0, s = 1", "ms": fx_ms,
                     "error_vs_exact_alibi": error_stats(fx_out, exact)}
        log(f"[bench] fixed blocks: {fx_ms:.3f} ms, rel. error vs exact {fixed_rec['error_vs_exact_alibi']['rel_fro']:.3f}"
            f" (estimator {err['rel_fro']:.3f})")
        del fx_out, ft

    # the unfused form (s single-sample passes writing fp32 partials, then a
    # log-sum-exp combine): what the sample fusion saves
    unfused_rec = None
    if not args.no_comparators:
        uf_out = torch.empty_like(qd)
        uf_ms, _ = time_calls(lambda: plsh.attention_unfused(qd, kd, vd, w.sigma, w.s, dt, causal=w.causal,
                                                              out=uf_out), 3, w.s)
        uf_diff = float((uf_out.float() - out.float()).abs().max())
        unfused_rec = {"ms": uf_ms, "over_fused_call": uf_ms / ms,
                       "partials_bytes": w.s * B * H * n * (d + 1) * 4,
                       "max_abs_diff_from_fused": uf_diff}
        log(f"[bench] unfused: {uf_ms:.3f} ms ({uf_ms / ms:.1f}x the fused call), max |diff| from fused {uf_diff:.3e}")
        del uf_out

    # the literal walk (one MFMA pass per sample with 0/1 masks inside one
    # kernel): the MFMA work the multiplicity fusion saves
    walk_rec = None
    if not args.no_comparators:
        wk_out = torch.empty_like(qd)
        wk_ms, wk_kernel_ms = time_calls(lambda: plsh.attention_walk(qd, kd, vd, w.sigma, w.s, dt, causal=w.causal,
                                                                    out=wk_out), 10)
        wk_diff = float((wk_out.float() - out.float()).abs().max())
        walk_rec = {"ms": wk_ms, "kernel_ms": wk_kernel_ms, "over_fused_call": wk_ms / ms,
                    "over_fused_kernel": wk_kernel_ms / kernel_ms,
                    "s_walk_tflops_in_kernel": f_alg / (wk_kernel_ms / 1e3) / 1e12,
                    "mfma_work_over_fused": pairs_alg / pairs_distinct,
                    "max_abs_diff_from_fused": wk_diff}
        log(f"[bench] walk: {wk_ms:.3f} ms ({wk_ms / ms:.1f}x the fused call; kernel {wk_kernel_ms:.3f} ms, "
            f"{walk_rec['s_walk_tflops_in_kernel']:.0f} TFLOP/s of s-walk work), max |diff| from fused {wk_diff:.3e}")
        del wk_out

    # the backward for fixed tables (the estimator's forward with each row's
    # normaliser, the dQ kernel, the dK/dV kernel): its call time; and the
    # backward from a saved forward, with the relative difference of the two
    # gradients (zero: the first runs the second after its own forward)
    bwd_rec = None
    if not args.no_comparators:
        g = torch.Generator().manual_seed(3)
        do = torch.randn(q.shape, generator=g).to(q.dtype)
        dod = do.to(dev)
        res = {}

        def bwd():
            res["g"] = plsh.attention_backward(qd, kd, vd, dod, w.sigma, w.s, dt, causal=w.causal)

        bw_ms, _ = time_calls(bwd, 10, 3)
        g_rec = res["g"]
        # the five products of a pair (S, dP, dV, dQ, dK; 10 d flops) count as useful
        bw_tflops = 2.5 * f_distinct / (bw_ms / 1e3) / 1e12
        bwd_rec = {"ms": bw_ms, "over_forward_call": bw_ms / ms, "useful_tflops": bw_tflops,
                   "useful_pct_bf16_peak": 100.0 * bw_tflops / PEAK_BF16_TFLOPS}
        log(f"[bench] backward: {bw_ms:.3f} ms ({bw_ms / ms:.1f}x the forward call, {bw_tflops:.0f} useful "
            f"TFLOP/s)")
        # the same backward from a saved forward (output and row normalisers of
        # plsh_alibi_attention_lse): no forward inside the call
        def bwd_saved():
            res["g"] = plsh.attention_backward(qd, kd, vd, dod, w.sigma, w.s, dt, causal=w.causal,
                                               out=o_s, lse2=l_s)

        bs_ms, _ = time_calls(bwd_saved, 10, 2)
        diffs = [float((a.float() - b.float()).abs().max() / b.float().abs().max())
                 for a, b in zip(res["g"], g_rec)]
        bwd_rec["saved_forward"] = {"forward_with_lse_ms": fl_ms, "forward_with_lse_kernel_ms": fl_kernel_ms,
                                    "backward_ms": bs_ms,
                                    "backward_over_recomputing": bs_ms / bw_ms,
                                    "rel_diff_from_recomputing_dq_dk_dv": diffs}
        log(f"[bench] saved forward: forward+lse {fl_ms:.3f} ms, backward {bs_ms:.3f} ms "
            f"({bs_ms / bw_ms:.2f}x the recomputing backward); rel. diff of dq, dk, dv "
            + ", ".join(f"{x:.1e}" for x in diffs))
        del dod, res, o_s, l_s, g_rec

    # the same shape at the other sample counts (s = 40: the n = 16k case whose
    # useful-FLOP target lies under the HBM roof)
    companions = []
    if not args.no_comparators and w.name.startswith("mistral-7b-n16384"):
        for other in ("mistral-7b-n16384-s10", "mistral-7b-n16384-s40"):
            if other != w.name:
                c = companion(other, 0.3)
                companions.append(c)
                log(f"[bench] {other}: {c['ms_per_call']:.4f} ms/call, kernel {c['kernel_ms']:.4f} ms, HBM frac "
                    f"{c['roofline']['frac']:.3f}, useful {c['roofline']['useful_pct_bf16_peak_in_kernel']:.1f}% "
                    f"of bf16 peak in the kernel (attainable {c['roofline']['attainable_pct_bf16_peak']:.1f}%)")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, q, k, v, tables, args.cpu_budget, out)
        log(f"[bench] cpu baseline {cpu['value']:.4g} rows*samples/s; max |gpu - oracle| on its heads "
            f"{cpu['parity_with_gpu_max_abs']:.3e}")

    rec = {
        "metric": "LSH-ALiBi attn query-rows\u00b7samples/s + useful MFMA TFLOP/s (% peak), n=16k",
        "value": rows_samples,
        "unit": "query-rows*samples/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_calls": settle_calls,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded Gaussian Q/K/V of the model's attention shape; no trained weights)",
        "config": {"workload": w.name, "batch": B, "heads": H, "kv_heads": Hkv, "n": n, "d": d,
                   "s": s, "causal": w.causal, "sigma": "ALiBi geometric slopes" if len(set(w.sigma)) > 1
                   else w.sigma[0], "heavy_tail_keys": w.heavy_tail, "parallelism": "single GPU"},
        "useful_tflops": useful_tflops,
        "useful_pct_bf16_peak": 100.0 * useful_tflops / PEAK_BF16_TFLOPS,
        "s_walk_equivalent_tflops": f_alg / sec / 1e12,
        "pairs_distinct": B * pairs_distinct,
        "pairs_alg": B * pairs_alg,
        "roofline": {**roofline_entry(w, pairs_distinct, kernel_ms, ms), "traffic": traffic,
                     "kernel": kernel_name(w),
                     "issued_pairs": issued,
                     "issued_tflops_in_kernel": 4.0 * d * issued / (kernel_ms / 1e3) / 1e12,
                     "mfma_counters": None if mfma_flops is None else {
                         "bf16_tflop_per_launch": mfma_flops / 1e12,
                         "tflops": mfma_flops / (kernel_ms / 1e3) / 1e12,
                         "pct_bf16_peak": 100.0 * mfma_flops / (kernel_ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS,
                         "source": "SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512, profiles/mfma.json"}},
        "timing": {"steps": {"ms_per_step": ms, "kernel_ms": kernel_ms, "mean_over": args.steps},
                   "warm": warm, "cold": cold, "graph_replay_ms_per_call": graph_ms,
                   "records_built_once_ms_per_call": rec_ms},
        "other_sample_counts": companions,
        "cpu_baseline": cpu,
        "host_sample_ms": host_sample_ms,
        "error_vs_exact_alibi": err,
        "exact_alibi_comparator": exact_rec,
        "fixed_blocks_baseline": fixed_rec,
        "unfused_ablation": unfused_rec,
        "walk_ablation": walk_rec,
        "backward": bwd_rec,
        "kernel_sha": kernel_sha(),
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
