#!/usr/bin/env python3
"""Benchmark of the Parallax attention hot path on one MI355X.

One step is one pass of the whole path over one batch of synthetic input:
  1. parallax_decode on the large decode workload: batch 256, 16 heads,
     head_dim 128, context 8192, bf16 (K + V = 17.18 GB streamed once);
  2. parallax_fwd on the bf16 causal prefill workload: batch 8, seq 4096,
     16 heads, head_dim 128, rho = x W_R (1.0998 TFLOP algorithmic);
  3. parallax_bwd, the backward of that prefill for a seeded dout
     (2.1996 TFLOP algorithmic: 16*D per causal pair);
  4. parallax_decode_gqa on the paged grouped-query decode workload: batch
     256, 32 query heads on 8 key-value heads, head_dim 128, context 8192,
     16-token pages in shuffled order (K + V = 8.59 GB streamed once);
  5. parallax_fwd_varlen on the packed causal prefill workload: 16
     sequences of 256..4096 tokens (40,827 in all), 16 heads, head_dim 128,
     rho = x W_R (1.0178 TFLOP algorithmic over the causal pairs);
  6. parallax_project, the fused q, k, v, rho input projection of the 1.7B
     shape: x [32768, 2048] times the stacked weight [8192, 2048], bf16
     (1.0995 TFLOP).
Inputs are seeded synthetic tensors already resident in HBM when the timed
region starts.

Reported (one JSON line on stdout):
  value           decode HBM throughput in GB/s: algorithmic bytes
                  (K + V of every visible position, q, rho, fp32 out) over
                  the decode kernel's average duration (HIP events on the
                  stream the kernels run on);
  prefill         TFLOP/s over the prefill kernel's average duration, with
                  algorithmic flops 8*D per causal (query, key) pair;
  roofline        decode kernel against 8 TB/s HBM;
  roofline_prefill prefill kernel against 2516.6 TFLOP/s dense bf16 MFMA;
  backward        TFLOP/s of one parallax_bwd call (all its kernels) with
                  algorithmic flops 16*D per causal pair (recomputed q.k and
                  rho.k, dout.v, dq, drho, two dk contractions, dv), and
                  roofline_backward against the same MFMA peak;
  backward_saved  the same backward from a training forward's saved tensors
                  (parallax_fwd_train run once before timing, then
                  parallax_bwd_saved: no second forward pass), same flops;
  prefill_varlen  TFLOP/s of the packed prefill and roofline_prefill_varlen
                  against the MFMA peak (flops 8*D per causal pair within
                  each sequence);
  project         TFLOP/s of the fused projection and roofline_project
                  against the MFMA peak (2 M N K flops);
  decode_gqa      GB/s of the paged grouped-query decode (K + V of every
                  visible position once per kv head, q, rho, fp32 out and
                  the block table) and roofline_decode_gqa against 8 TB/s;
  decode_softmax_only, hbm_read_reference
                  context, outside the step: parallax_decode with rho = NULL
                  (plain softmax attention: same bytes, half the arithmetic)
                  and parallax_stream_read over the same K and V bytes (the
                  plain read rate of HBM on this GPU);
  decode_small    context, outside the step: the one-sequence decode
                  (batch 1, 16 heads, context 4096) cycling 16 input copies
                  so each launch reads from HBM (latency-bound point);
  cpu_baseline    the fp64 oracle timed on the host's cores on a bounded
                  sample of the decode workload; cpu_baseline_<row> the same
                  for the other rows (prefill, backward, decode_gqa,
                  prefill_varlen, project), inputs converted to fp64 before
                  the timed region;
  ms_min, ms_median
                  per row, the fastest and the median of its timed launches
                  (ms is their mean);
  sustained_gfx_clock_mhz
                  under prefill: the graphics clock (mean over the XCDs, read
                  with amd-smi) while the prefill runs back to back after the
                  timed region, and the prefill's fraction of the MFMA peak
                  rescaled to that clock (the peak is quoted at 2.4 GHz);
  device          name, architecture, compute units and maximum graphics
                  clock of the GPU.

``--lla`` compares with exact Local Linear Attention: the oracle solves the
per-query probe (S_i + lam I)^-1 (kbar_i - q_i) by conjugate gradient on the
host (the solve Parallax replaces), and parallax_fwd then runs once with
that probe on the GPU; one JSON line reports the solve's time and key
passes against the single pass.

``--sweep-gqa`` times the paged and contiguous grouped-query decode (32 query
heads on 8 kv heads, head_dim 128, 16-token pages) over batch x context.

Other modes: ``--sweep`` times the decode grid (batch x context, uniform and
ragged lengths) and prints one JSON line per point. ``--copy-calibration``
runs one plain device copy of 1 GiB (the known-size kernel used to scale
memory counters).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("decode KV GB/s + % HBM peak; prefill TFLOP/s + % MFMA peak "
          "(1 GPU)")
HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2516.6  # 256 CU x 4096 flop/clk x 2.4 GHz, dense
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "traffic.json")
CSRC = os.path.join(ROOT, "transformer_attention_parallax_amd", "csrc")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-clock", action="store_true",
                    help="query no clocks with amd-smi (neither the graphics clock under "
                         "the prefill load nor the device maximum); use under a profiler")
    ap.add_argument("--no-reference", action="store_true",
                    help="skip the softmax-only decode and plain-read reference rows")
    ap.add_argument("--only", choices=["decode", "prefill", "backward", "backward_saved",
                                       "decode_gqa", "prefill_varlen", "project",
                                       "decode_small", "prefill_f32"], default=None)
    ap.add_argument("--sweep", action="store_true")
    ap.add_argument("--sweep-max-tokens", type=int, default=1 << 24)
    ap.add_argument("--sweep-batches", type=str, default=None,
                    help="comma-separated batch sizes of the sweep to run (default: all)")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--sweep-gqa", action="store_true")
    ap.add_argument("--lla", action="store_true",
                    help="exact local-linear probe (host CG) against one Parallax pass")
    ap.add_argument("--lla-lam", type=float, default=1.0)
    ap.add_argument("--with-copy", action="store_true",
                    help="also run one 1 GiB device copy before timing (the "
                         "known-size kernel that scales memory counters)")
    return ap.parse_args()


def source_hash(*files) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic_for(kernel: str, src_files, launches_bytes_key="bytes_per_launch"):
    """HBM bytes per launch measured by counters, if still current."""
    try:
        with open(PROFILE_TRAFFIC) as f:
            rec = json.load(f).get(kernel)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha256") != source_hash(*src_files):
        return None
    return rec.get(launches_bytes_key)


def decode_bytes(B, H, D, seqlens, in_bytes=2, out_bytes=4):
    tokens = int(sum(int(x) for x in seqlens))
    return tokens * H * 2 * D * in_bytes + B * H * D * (2 * in_bytes + out_bytes)


def decode_gqa_bytes(B, Hq, Hkv, D, L, page, in_bytes=2, out_bytes=4):
    npb = (L + page - 1) // page
    return (B * L * Hkv * 2 * D * in_bytes + B * Hq * D * (2 * in_bytes + out_bytes)
            + B * npb * 4)


def prefill_flops(B, N, H, D):
    return 8 * D * B * H * N * (N + 1) // 2


def backward_flops(B, N, H, D):
    return 16 * D * B * H * N * (N + 1) // 2


def cpu_count() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def cpu_model() -> str:
    """The host CPU's model name (first entry of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline_whole_decode(inp, gpu_out, tol=2e-2):
    """Time the fp64 oracle on a whole (small) decode workload: every (b, h)
    stream at its full length; the result is also compared with the GPU's."""
    import numpy as np
    import oracle
    q, rho, k, v, sl = (inp[n] for n in ("q", "rho", "k", "v", "seqlens"))
    B, H, L, D = k.shape
    qs, rs, ks, vs = (x.double().cpu().numpy() for x in (q, rho, k, v))
    sls = sl.cpu().numpy()
    t0 = time.perf_counter()
    ref = oracle.decode(qs, rs, ks, vs, seqlens=sls, scale=1.0 / math.sqrt(D))
    t = time.perf_counter() - t0
    err = float(np.abs(gpu_out.double().cpu().numpy() - ref).max())
    nbytes = decode_bytes(B, H, D, sls.tolist())
    return {"value": nbytes / t / 1e9, "unit": "GB/s", "cores": oracle.max_threads(),
            "kind": "oracle", "max_abs_err_vs_gpu": err, "tol": tol,
            "sample": f"the whole workload (B{B} H{H} D{D} L{L}, every stream); "
                      f"{t:.3f} s; explicit fp64 covariance per query"}


def cpu_baseline_whole_prefill(inp, gpu_out, tol):
    """Time the fp64 oracle on a whole (small) causal prefill workload."""
    import numpy as np
    import oracle
    q, k, v, rho = (inp[n] for n in ("q", "k", "v", "rho"))
    B, N, H, D = q.shape
    qc, kc, vc, rc = (x.double().cpu().numpy() for x in (q, k, v, rho))
    t0 = time.perf_counter()
    ref = oracle.fwd(qc, kc, vc, rc, causal=True, scale=1.0 / math.sqrt(D))
    t = time.perf_counter() - t0
    err = float(np.abs(gpu_out.double().cpu().numpy() - ref).max())
    return {"value": prefill_flops(B, N, H, D) / t / 1e12, "unit": "TFLOP/s",
            "cores": oracle.max_threads(), "kind": "oracle",
            "max_abs_err_vs_gpu": err, "tol": tol,
            "sample": f"the whole workload (B{B} N{N} H{H} D{D}, every query row); "
                      f"{t:.3f} s; explicit fp64 covariance per row"}


def cpu_baseline_decode(inp, gpu_out, target_s=12.0):
    """Time the fp64 oracle on a bounded sample of (b, h) streams; the timed
    sample's outputs are also compared with the GPU's (gpu_out)."""
    import numpy as np
    import oracle
    q, rho, k, v = inp["q"], inp["rho"], inp["k"], inp["v"]
    B, H, L, D = k.shape
    order = [(b, h) for b in range(B) for h in range(H)]
    rng = np.random.default_rng(7)
    order = [order[i] for i in rng.permutation(len(order))]

    def sample(n):
        sel = order[:n]
        qs = np.stack([q[b, h].double().cpu().numpy() for b, h in sel])[:, None]
        rs = np.stack([rho[b, h].double().cpu().numpy() for b, h in sel])[:, None]
        ks = np.stack([k[b, h].double().cpu().numpy() for b, h in sel])[:, None]
        vs = np.stack([v[b, h].double().cpu().numpy() for b, h in sel])[:, None]
        t0 = time.perf_counter()
        ref = oracle.decode(qs, rs, ks, vs, scale=1.0 / math.sqrt(D))
        dt = time.perf_counter() - t0
        got = np.stack([gpu_out[b, h].double().cpu().numpy() for b, h in sel])
        return dt, float(np.abs(got - ref[:, 0]).max())

    n0 = 16
    t_probe, _ = sample(n0)
    n = int(min(len(order), max(n0, round(n0 * target_s / max(t_probe, 1e-3)))))
    t, err = sample(n)
    gb = n * L * D * 2 * 2 / 1e9  # bf16 K + V bytes of the sampled streams
    return {"value": gb / t, "unit": "GB/s", "cores": oracle.max_threads(),
            "kind": "oracle", "max_abs_err_vs_gpu": err, "tol": 2e-2,
            "sample": f"{n} of {B * H} (b, h) streams of the decode workload, "
                      f"full {L}-key context each; {t:.1f} s; explicit fp64 "
                      f"covariance per query; host has {cpu_count()} cores"}


def cpu_baseline_prefill(inp, gpu_out, target_s=10.0):
    import numpy as np
    import oracle
    q, k, v, rho = (inp[n] for n in ("q", "k", "v", "rho"))
    B, N, H, D = q.shape
    rng = np.random.default_rng(8)
    bsel = 0
    qc, kc, vc, rc = (x[bsel:bsel + 1].double().cpu().numpy() for x in (q, k, v, rho))

    def sample(n):
        rows = [(0, int(i), int(h)) for i, h in
                zip(rng.integers(0, N, n), rng.integers(0, H, n))]
        t0 = time.perf_counter()
        ref = oracle.fwd_rows(qc, kc, vc, rc, rows, causal=True)
        dt = time.perf_counter() - t0
        flops = sum(8 * D * (i + 1) for _, i, _ in rows)
        got = np.stack([gpu_out[bsel, i, h].double().cpu().numpy() for _, i, h in rows])
        return dt, flops, float(np.abs(got - ref).max())

    t_probe, _, _ = sample(32)
    n = int(max(32, round(32 * target_s / max(t_probe, 1e-3))))
    t, flops, err = sample(n)
    return {"value": flops / t / 1e12, "unit": "TFLOP/s",
            "cores": oracle.max_threads(), "kind": "oracle",
            "max_abs_err_vs_gpu": err, "tol": 2e-2,
            "sample": f"{n} random (i, h) query rows of batch 0 of the prefill "
                      f"workload; {t:.1f} s; explicit fp64 covariance per row"}


def _blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [d.get("num_threads", 0) for d in threadpool_info() if d.get("user_api") == "blas"]
        return max(n) if n else cpu_count()
    except Exception:   # threadpoolctl absent or unreadable
        return cpu_count()


def cpu_baseline_backward(inp, dout, gpu_grads, target_s=10.0):
    """Time the fp64 backward oracle on whole (b, h) heads of the backward
    workload (every causal pair of each sampled head); each sampled head's
    gradients are also compared with the GPU's, relative to the largest
    oracle entry of that gradient."""
    import numpy as np
    import oracle
    q, k, v, rho = (inp[n] for n in ("q", "k", "v", "rho"))
    B, N, H, D = q.shape
    rng = np.random.default_rng(9)
    heads = [(i // H, i % H) for i in rng.permutation(B * H)]

    rel = [0.0]

    def run(sel):
        t = 0.0
        for b, h in sel:
            xs = [x[b:b + 1, :, h:h + 1].double().cpu().numpy() for x in (q, k, v, rho, dout)]
            t0 = time.perf_counter()
            refs = oracle.bwd(*xs, causal=True)
            t += time.perf_counter() - t0
            for g, ref in zip(gpu_grads, refs):
                got = g[b:b + 1, :, h:h + 1].double().cpu().numpy()
                rel[0] = max(rel[0], float(np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30)))
        return t

    t = run(heads[:1])
    n = int(max(1, min(len(heads), round(target_s / max(t, 1e-3)))))
    t += run(heads[1:n])
    flops = n * backward_flops(1, N, 1, D)
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": oracle.max_threads(),
            "kind": "oracle", "max_rel_err_vs_gpu": rel[0], "tol_rel": 1e-2,
            "sample": f"{n} of {B * H} whole (b, h) heads of the backward workload "
                      f"({N} tokens, all causal pairs); {t:.1f} s; fp64"}


def cpu_baseline_decode_gqa(inp, gpu_out, target_s=8.0):
    """Time the fp64 decode oracle on sampled (b, kv head) streams of the
    paged grouped-query workload, all query heads of each, gathered from the
    pages first (outside the timing)."""
    import numpy as np
    import oracle
    q, rho, k, v, bt = inp["q"], inp["rho"], inp["k"], inp["v"], inp["block_table"]
    B, Hq, D = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    L = int(inp["seqlens"][0])
    rng = np.random.default_rng(10)
    pairs = [(i // Hkv, i % Hkv) for i in rng.permutation(B * Hkv)]

    err = [0.0]

    def run(sel):
        t = 0.0
        for b, hk in sel:
            pages = bt[b].long()
            kk = k[pages, :, hk, :].reshape(-1, D)[:L]
            vv = v[pages, :, hk, :].reshape(-1, D)[:L]
            qs = q[b, hk * G:(hk + 1) * G].double().cpu().numpy()[None]
            rs = rho[b, hk * G:(hk + 1) * G].double().cpu().numpy()[None]
            ks = kk.double().cpu().numpy()[None, None].repeat(G, axis=1)
            vs = vv.double().cpu().numpy()[None, None].repeat(G, axis=1)
            t0 = time.perf_counter()
            ref = oracle.decode(qs, rs, ks, vs, scale=1.0 / math.sqrt(D))
            t += time.perf_counter() - t0
            got = gpu_out[b, hk * G:(hk + 1) * G].double().cpu().numpy()
            err[0] = max(err[0], float(np.abs(got - ref[0]).max()))
        return t

    t = run(pairs[:2])
    n = int(max(2, min(len(pairs), round(2 * target_s / max(t, 1e-3)))))
    t += run(pairs[2:n])
    gb = n * L * D * 2 * 2 / 1e9  # bf16 K + V of the sampled kv streams, once each
    return {"value": gb / t, "unit": "GB/s", "cores": oracle.max_threads(), "kind": "oracle",
            "max_abs_err_vs_gpu": err[0], "tol": 2e-2,
            "sample": f"{n} of {B * Hkv} (b, kv head) streams of the paged grouped-query "
                      f"workload, {G} query heads each, full {L}-key context; {t:.1f} s; "
                      f"explicit fp64 covariance per query"}


def cpu_baseline_prefill_varlen(inp, lens, gpu_out, target_s=8.0):
    """Time the fp64 oracle on random query rows of the packed prefill
    workload (rows drawn over all tokens, each against its own sequence)."""
    import numpy as np
    import oracle
    q, k, v, rho = (inp[n] for n in ("q", "k", "v", "rho"))
    T, H, D = q.shape
    starts = np.concatenate([[0], np.cumsum(lens)])
    seqs = [tuple(x[int(starts[b]):int(starts[b + 1])].double().cpu().numpy()[None]
                  for x in (q, k, v, rho)) for b in range(len(lens))]
    rng = np.random.default_rng(11)

    def run(n):
        toks = rng.integers(0, T, n)
        bs = np.searchsorted(starts, toks, side="right") - 1
        hs = rng.integers(0, H, n)
        t, flops, err = 0.0, 0, 0.0
        for b in np.unique(bs):
            sel = np.nonzero(bs == b)[0]
            rows = [(0, int(toks[j] - starts[b]), int(hs[j])) for j in sel]
            t0 = time.perf_counter()
            ref = oracle.fwd_rows(*seqs[b], rows, causal=True)
            t += time.perf_counter() - t0
            flops += sum(8 * D * (i + 1) for _, i, _ in rows)
            got = np.stack([gpu_out[int(starts[b]) + i, h].double().cpu().numpy()
                            for _, i, h in rows])
            err = max(err, float(np.abs(got - ref).max()))
        return t, flops, err

    # per-sequence calls make small samples overhead-bound: grow the sample
    # until it takes at least half the target time
    n = 64
    t, flops, err = run(n)
    while t < 0.5 * target_s and n < (1 << 20):
        n = int(n * min(8.0, max(2.0, target_s / max(t, 1e-3))))
        t, flops, err = run(n)
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": oracle.max_threads(),
            "kind": "oracle", "max_abs_err_vs_gpu": err, "tol": 2e-2,
            "sample": f"{n} random (token, head) query rows of the packed prefill workload "
                      f"({len(lens)} sequences); {t:.1f} s; explicit fp64 covariance per row"}


def cpu_baseline_project(inp, gpu_out, target_s=8.0):
    """Time the fp64 projection oracle (one library matrix product) on a
    sample of rows of x; the timed sample is also compared with the GPU's
    bf16 output, element by element against one bf16 rounding plus fp32
    accumulation in another order."""
    import numpy as np
    import oracle
    x, w = inp["x"], inp["w"]
    M, K = x.shape
    N = w.shape[0]
    wf = w.double().cpu().numpy()
    rng = np.random.default_rng(12)

    def run(m):
        rows = np.sort(rng.choice(M, m, replace=False))
        idx = torch_index(rows, x.device)
        xs = x[idx].double().cpu().numpy()
        t0 = time.perf_counter()
        ref = oracle.project(xs, wf)
        dt = time.perf_counter() - t0
        got = gpu_out[idx].double().cpu().numpy()
        err = np.abs(got - ref)
        bound = 2.0 ** -8 * np.abs(ref) + 2.0 ** -16 * (np.abs(xs) @ np.abs(wf).T)
        return dt, float(err.max()), bool((err <= bound).all())

    t, _, _ = run(64)
    m = int(min(M, max(64, round(64 * target_s / max(t, 1e-3)))))
    t, err, ok = run(m)
    return {"value": 2 * m * N * K / t / 1e12, "unit": "TFLOP/s", "cores": _blas_threads(),
            "kind": "oracle", "max_abs_err_vs_gpu": err, "within_bound": ok,
            "bound": "2^-8 |ref| + 2^-16 sum_k |x_k w_k| per element",
            "sample": f"{m} of {M} random rows of x against the full stacked weight "
                      f"[{N}, {K}]; {t:.1f} s; fp64 library product"}


def torch_index(rows, device):
    import torch
    return torch.as_tensor(rows, dtype=torch.long, device=device)


def _amd_smi_clocks():
    """(current, max) graphics clock in MHz, each averaged over the XCDs, from
    one `amd-smi metric -c --json` call (a child process); None if absent."""
    import shutil
    import subprocess
    exe = shutil.which("amd-smi")
    if exe is None:
        return None
    try:
        out = subprocess.run([exe, "metric", "-c", "--json"], capture_output=True,
                             text=True, timeout=20).stdout
        data = json.loads(out)
    except (OSError, ValueError, subprocess.SubprocessError):
        return None
    gpus = data.get("gpu_data", data) if isinstance(data, dict) else data
    if not gpus:
        return None
    clk = gpus[0].get("clock", {})
    cur = [v["clk"]["value"] for k, v in clk.items()
           if k.startswith("gfx") and isinstance(v.get("clk", {}).get("value"), (int, float))]
    mx = [v["max_clk"]["value"] for k, v in clk.items()
          if k.startswith("gfx") and isinstance(v.get("max_clk", {}).get("value"), (int, float))]
    if not cur:
        return None
    return sum(cur) / len(cur), (sum(mx) / len(mx) if mx else None)


def sustained_clock(torch, fn, seconds=1.5):
    """Mean graphics clock (MHz) read while `fn` runs back to back on the GPU
    (outside any timed region); None if amd-smi is not available."""
    import threading
    readings = []
    stop = threading.Event()

    def poll():
        while not stop.is_set():
            r = _amd_smi_clocks()
            if r is None:
                return
            readings.append(r[0])

    th = threading.Thread(target=poll, daemon=True)
    fn()
    torch.cuda.synchronize()
    th.start()
    t0 = time.perf_counter()
    while th.is_alive() and (time.perf_counter() - t0 < seconds or
                             (not readings and time.perf_counter() - t0 < 30.0)):
        for _ in range(4):
            fn()
        torch.cuda.synchronize()
    stop.set()
    th.join(timeout=30.0)
    return round(sum(readings) / len(readings), 1) if readings else None


def time_events(torch, fns, steps, warmup, stream, min_warmup_s=1.0,
                row_warmup_s=0.1, samples=None):
    """Time `steps` passes of every fn; returns (wall_s, per-fn mean seconds).

    Each fn (one row of the path) runs its `steps` launches back to back,
    bracketed by HIP events per launch on `stream`, inside a synchronised
    region of its own; wall_s sums those regions, which together hold exactly
    `steps` passes of the whole path. Before each row's region the row runs
    untimed for `row_warmup_s`: on this GPU the compute clock drops during a
    memory-bound kernel and takes about a millisecond to come back, which
    would otherwise be charged to the first launches of the next row.

    Untimed global warmup first: at least `warmup` steps and at least
    `min_warmup_s` seconds. If `samples` is a list, it receives each fn's
    per-launch durations in seconds."""
    t0 = time.perf_counter()
    done = 0
    while done < warmup or time.perf_counter() - t0 < min_warmup_s:
        for fn in fns:
            fn()
        done += 1
        if done % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)] for _ in fns]
    wall = 0.0
    for i, fn in enumerate(fns):
        t0 = time.perf_counter()
        n = 0
        while n < 2 or time.perf_counter() - t0 < row_warmup_s:
            fn()
            n += 1
            if n % 4 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(steps):
            ev[i][s][0].record(stream)
            fn()
            ev[i][s][1].record(stream)
        torch.cuda.synchronize()
        wall += time.perf_counter() - t0
    dur = [[a.elapsed_time(b) / 1e3 for a, b in ev[i]] for i in range(len(fns))]
    if samples is not None:
        samples.extend(dur)
    per = [sum(d) / steps for d in dur]
    return wall, per


_SLEEP_RATE = []


def gpu_sleep(torch, stream, seconds):
    """Hold `stream` for about `seconds` with a spinning kernel, so that the
    host can enqueue the launches that follow before the GPU reaches them.
    The spin rate (cycles per second) is measured once with HIP events."""
    if not _SLEEP_RATE:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(1000)
        a.record(stream)
        torch.cuda._sleep(2_000_000)
        b.record(stream)
        torch.cuda.synchronize()
        _SLEEP_RATE.append(2_000_000 / (a.elapsed_time(b) / 1e3))
    torch.cuda._sleep(int(seconds * _SLEEP_RATE[0]))


def time_queued(torch, fn, steps, stream, host_s_per_call):
    """Per-launch GPU durations of `steps` launches of `fn` enqueued while
    the stream is held by a spin, so no launch waits for the host: events
    then time the GPU's own work (kernel plus dispatch), not the host's
    submission rate. Returns the list of durations in seconds."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    gpu_sleep(torch, stream, 2.0 * steps * host_s_per_call + 2e-3)
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) / 1e3 for a, b in ev]


def time_back_to_back(torch, fn, steps, stream, host_s_per_call):
    """Mean GPU time per call of `steps` calls of `fn` run back to back: the
    calls are enqueued behind a GPU spin and bracketed by one pair of HIP
    events, so the per-call time holds each call's own launches and their
    dispatch but not the event packets between calls."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    gpu_sleep(torch, stream, 2.0 * steps * host_s_per_call + 2e-3)
    a.record(stream)
    for _ in range(steps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / 1e3 / steps


def time_graph(torch, step, calls, stream, replays=20):
    """Seconds per call when `calls` calls of `step` are captured in one HIP
    graph (torch.cuda.graph) and the graph is replayed back to back."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(calls):
            step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(calls):
            step()
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(replays):
        graph.replay()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / 1e3 / (replays * calls)


def run_small(args):
    """The two latency-bound context rows alone (--only decode_small or
    --only prefill_f32), with their oracle baselines: one JSON line."""
    import torch
    import transformer_attention_parallax_amd as px

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    if args.with_copy:
        run_copy_calibration()
    keep = {}
    if args.only == "decode_small":
        row = decode_small_row(torch, px, stream, args.steps, keep=keep)
        val, unit = row["decode_small"]["gbps"], "GB/s"
    else:
        row = prefill_f32_row(torch, px, stream, args.steps, keep=keep)
        val, unit = row["prefill_f32"]["tflops"], "TFLOP/s"
    line = {"metric": METRIC, "value": round(val, 3), "unit": unit, "n_gpus": 1,
            "steps": args.steps, "config": {"workload": row[args.only]["workload"]}}
    line.update(row)
    if not args.no_cpu_baseline:
        inp, out = keep[args.only]
        res = (cpu_baseline_whole_decode(inp, out) if args.only == "decode_small"
               else cpu_baseline_whole_prefill(inp, out, tol=1e-4))
        res["cpu_model"] = cpu_model()
        res["host_cores"] = cpu_count()
        line["cpu_baseline"] = res
    print(json.dumps(line), flush=True)


def run_main(args):
    import torch
    import synth
    import transformer_attention_parallax_amd as px

    if args.only in ("decode_small", "prefill_f32"):
        return run_small(args)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    fns, names = [], []
    dec = pre = None
    if args.only in (None, "decode"):
        dshp = synth.WORKLOADS["decode_large"]
        dec = synth.decode_inputs(dshp, device=dev)
        dec_out = torch.empty((dshp.B, dshp.H, dshp.D), device=dev)
        ws_bytes = px.decode_workspace_size(dshp.B, dshp.H, dshp.D, dshp.L)
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
        fns.append(lambda: px.decode(dec["q"], dec["k"], dec["v"], dec["rho"],
                                     dec["seqlens"], out=dec_out, workspace=ws))
        names.append("decode")
    if args.only in (None, "prefill"):
        pshp = synth.WORKLOADS["prefill_bf16"]
        pre = synth.prefill_inputs(pshp, device=dev)
        pre_out = torch.empty((pshp.B, pshp.N, pshp.H, pshp.D), device=dev)
        pre_ws = torch.empty(px.fwd_workspace_size(pshp.B, pshp.N, pshp.H, pshp.D),
                             dtype=torch.uint8, device=dev)
        fns.append(lambda: px.fwd(pre["q"], pre["k"], pre["v"], pre["rho"],
                                  causal=True, out=pre_out, workspace=pre_ws))
        names.append("prefill")
    bwd = None
    if args.only in (None, "backward"):
        bshp = synth.WORKLOADS["prefill_bf16"]
        bwd = pre if pre is not None else synth.prefill_inputs(bshp, device=dev)
        g = synth.gen(1000 * bshp.index + 6, dev)
        bwd_dout = torch.randn(bwd["q"].shape, device=dev, generator=g).to(torch.bfloat16)
        bwd_grads = [torch.empty(bwd["q"].shape, device=dev) for _ in range(4)]
        bwd_ws = torch.empty(px.bwd_workspace_size(bshp.B, bshp.N, bshp.H, bshp.D),
                             dtype=torch.uint8, device=dev)
        fns.append(lambda: px.bwd(bwd["q"], bwd["k"], bwd["v"], bwd["rho"], bwd_dout,
                                  causal=True, grads=bwd_grads, workspace=bwd_ws))
        names.append("backward")
    bsv = None
    if args.only in (None, "backward_saved"):
        bshp = synth.WORKLOADS["prefill_bf16"]
        bsv = pre if pre is not None else (bwd if bwd is not None else
                                           synth.prefill_inputs(bshp, device=dev))
        g = synth.gen(1000 * bshp.index + 6, dev)
        bsv_dout = torch.randn(bsv["q"].shape, device=dev, generator=g).to(torch.bfloat16)
        bsv_out, bsv_vbar, bsv_lr = px.fwd_train(bsv["q"], bsv["k"], bsv["v"], bsv["rho"],
                                                 causal=True)
        bsv_grads = [torch.empty(bsv["q"].shape, device=dev) for _ in range(4)]
        bsv_ws = torch.empty(px.bwd_workspace_size(bshp.B, bshp.N, bshp.H, bshp.D),
                             dtype=torch.uint8, device=dev)
        fns.append(lambda: px.bwd_saved(bsv["q"], bsv["k"], bsv["v"], bsv["rho"], bsv_dout,
                                        bsv_out, bsv_vbar, bsv_lr, causal=True,
                                        grads=bsv_grads, workspace=bsv_ws))
        names.append("backward_saved")
    gqa = None
    if args.only in (None, "decode_gqa"):
        gshp = synth.WORKLOADS["decode_gqa_paged"]
        gqa = synth.paged_decode_inputs(gshp, device=dev)
        gqa_out = torch.empty((gshp.B, gshp.Hq, gshp.D), device=dev)
        gqa_ws = torch.zeros(max(1, px.decode_gqa_workspace_size(
            gshp.B, gshp.Hq, gshp.Hkv, gshp.D, gshp.L, paged=True)), dtype=torch.uint8,
            device=dev)
        fns.append(lambda: px.decode_gqa(gqa["q"], gqa["k"], gqa["v"], gqa["rho"],
                                         seqlens=gqa["seqlens"],
                                         block_table=gqa["block_table"],
                                         out=gqa_out, workspace=gqa_ws))
        names.append("decode_gqa")
    vl = None
    if args.only in (None, "prefill_varlen"):
        vshp = synth.WORKLOADS["prefill_varlen"]
        vl = synth.varlen_prefill_inputs(vshp, device=dev)
        vl_out = torch.empty(vl["q"].shape, device=dev)
        vl_ws = torch.empty(px.fwd_workspace_size(vshp.B, vshp.max_seqlen, vshp.H, vshp.D),
                            dtype=torch.uint8, device=dev)
        fns.append(lambda: px.fwd_varlen(vl["q"], vl["k"], vl["v"], vl["rho"],
                                         vl["cu_seqlens"], vshp.max_seqlen, causal=True,
                                         out=vl_out, workspace=vl_ws))
        names.append("prefill_varlen")
    prj = None
    if args.only in (None, "project"):
        jshp = synth.WORKLOADS["project_qkvr"]
        prj = synth.project_inputs(jshp, device=dev)
        prj_out = torch.empty((jshp.M, jshp.N), dtype=torch.bfloat16, device=dev)
        fns.append(lambda: px.project(prj["x"], prj["w"], out=prj_out))
        names.append("project")
    torch.cuda.synchronize()
    if args.with_copy:
        run_copy_calibration()

    samples = []
    wall, per = time_events(torch, fns, args.steps, args.warmup, stream, samples=samples)
    # the decode output is reused by the reference rows below; keep this one
    dec_snap = dec_out.clone() if dec is not None else None
    t = dict(zip(names, per))
    spread = {n: {"ms_min": min(d) * 1e3, "ms_median": statistics.median(d) * 1e3}
              for n, d in zip(names, samples)}
    # graphics clock under the prefill load, sampled after the timed region
    clock_mhz = None
    if "prefill" in names and not args.no_clock:
        clock_mhz = sustained_clock(torch, fns[names.index("prefill")])
    line = {"metric": METRIC, "value": None, "unit": "GB/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": wall / args.steps * 1e3, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded N(0,1) q/k/v; rho N(0,0.1^2) for "
                    "decode, rho = x W_R for prefill)",
            "config": {"workload": "", "parallelism": "none (1 GPU)"}}
    props = torch.cuda.get_device_properties(dev)
    clocks = None if args.no_clock else _amd_smi_clocks()
    line["device"] = {"name": props.name, "arch": getattr(props, "gcnArchName", None),
                      "compute_units": props.multi_processor_count,
                      "max_gfx_clock_mhz": clocks[1] if clocks else None}
    work = []
    if dec is not None:
        dshp = synth.WORKLOADS["decode_large"]
        nbytes = decode_bytes(dshp.B, dshp.H, dshp.D, dec["seqlens"].tolist())
        gbps = nbytes / t["decode"] / 1e9
        work.append(f"decode B{dshp.B} H{dshp.H} D{dshp.D} L{dshp.L} bf16 "
                    f"({nbytes / 1e9:.2f} GB/launch)")
        line["value"] = round(gbps, 2)
        line["decode"] = {"ms": t["decode"] * 1e3, "gbps": gbps,
                          "frac_hbm_peak": gbps / HBM_PEAK_GBPS,
                          "bytes_per_launch": nbytes,
                          "splits": px.decode_splits(dshp.B, dshp.H, dshp.D,
                                                     dshp.L)}
        line["roofline"] = {
            "bound": "hbm", "achieved": round(gbps, 2), "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4),
            "traffic": traffic_for("decode", ["decode.hip", "decode_common.h"]),
            "kernel": "decode_kernel<bf16, D=128, single split>"}
    if pre is not None:
        pshp = synth.WORKLOADS["prefill_bf16"]
        flops = prefill_flops(pshp.B, pshp.N, pshp.H, pshp.D)
        tf = flops / t["prefill"] / 1e12
        work.append(f"causal prefill B{pshp.B} N{pshp.N} H{pshp.H} D{pshp.D} "
                    f"bf16 ({flops / 1e12:.4f} TFLOP/launch)")
        line["prefill"] = {"ms": t["prefill"] * 1e3, "tflops": tf,
                           "frac_mfma_peak": tf / MFMA_BF16_PEAK_TFLOPS,
                           "flops_per_launch": flops}
        if clock_mhz:
            # the peak is quoted at 2.4 GHz; the same fraction at the clock
            # the chip actually held while running this row
            line["prefill"]["sustained_gfx_clock_mhz"] = clock_mhz
            line["prefill"]["frac_of_peak_at_sustained_clock"] = round(
                tf / (MFMA_BF16_PEAK_TFLOPS * clock_mhz / 2400.0), 4)
        line["roofline_prefill"] = {
            "bound": "mfma", "achieved": round(tf, 2),
            "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": traffic_for("prefill", ["fwd_mfma.hip", "pack.hip"]),
            "kernel": "parallax_fwd call: pack_t_kernel<128,64> (V to fp16 tiles) + "
                      "fwd_mfma_kernel<D=128, 4 waves> (bf16 in, 16x16x32 MFMA)"}
        if dec is None:
            line["value"] = round(tf, 2)
            line["unit"] = "TFLOP/s"
            line["roofline"] = line.pop("roofline_prefill")
    if bwd is not None:
        bshp = synth.WORKLOADS["prefill_bf16"]
        flops = backward_flops(bshp.B, bshp.N, bshp.H, bshp.D)
        tf = flops / t["backward"] / 1e12
        work.append(f"prefill backward B{bshp.B} N{bshp.N} H{bshp.H} D{bshp.D} "
                    f"bf16 ({flops / 1e12:.4f} TFLOP/call)")
        line["backward"] = {"ms": t["backward"] * 1e3, "tflops": tf,
                            "frac_mfma_peak": tf / MFMA_BF16_PEAK_TFLOPS,
                            "flops_per_call": flops}
        line["roofline_backward"] = {
            "bound": "mfma", "achieved": round(tf, 2),
            "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": traffic_for("backward", ["bwd_mfma.hip"]),
            "kernel": "parallax_bwd call: statistics pass (bwd_dq_kernel statistics "
                      "mode) + bwd_dq_kernel + bwd_dkv_kernel"}
        if dec is None and pre is None:
            line["value"] = round(tf, 2)
            line["unit"] = "TFLOP/s"
            line["roofline"] = line.pop("roofline_backward")
    if bsv is not None:
        bshp = synth.WORKLOADS["prefill_bf16"]
        flops = backward_flops(bshp.B, bshp.N, bshp.H, bshp.D)
        tf = flops / t["backward_saved"] / 1e12
        work.append(f"prefill backward from saved forward tensors B{bshp.B} N{bshp.N} "
                    f"H{bshp.H} D{bshp.D} bf16")
        line["backward_saved"] = {"ms": t["backward_saved"] * 1e3, "tflops": tf,
                                  "frac_mfma_peak": tf / MFMA_BF16_PEAK_TFLOPS,
                                  "flops_per_call": flops}
        line["roofline_backward_saved"] = {
            "bound": "mfma", "achieved": round(tf, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": traffic_for("backward_saved", ["bwd_mfma.hip"]),
            "kernel": "parallax_bwd_saved call: saved_stats_kernel + bwd_dq_kernel + "
                      "bwd_dkv_kernel"}
    if gqa is not None:
        gshp = synth.WORKLOADS["decode_gqa_paged"]
        nbytes = decode_gqa_bytes(gshp.B, gshp.Hq, gshp.Hkv, gshp.D, gshp.L, gshp.page)
        gbps = nbytes / t["decode_gqa"] / 1e9
        work.append(f"paged GQA decode B{gshp.B} Hq{gshp.Hq} Hkv{gshp.Hkv} D{gshp.D} "
                    f"L{gshp.L} page{gshp.page} bf16 ({nbytes / 1e9:.2f} GB/launch)")
        line["decode_gqa"] = {"ms": t["decode_gqa"] * 1e3, "gbps": gbps,
                              "frac_hbm_peak": gbps / HBM_PEAK_GBPS,
                              "bytes_per_launch": nbytes}
        line["roofline_decode_gqa"] = {
            "bound": "hbm", "achieved": round(gbps, 2), "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4),
            "traffic": traffic_for("decode_gqa", ["decode_gqa.hip", "decode_common.h"]),
            "kernel": "decode_gqa_kernel<D=128, G=4, paged, single split>"}
        if dec is None and pre is None and bwd is None:
            line["value"] = round(gbps, 2)
            line["roofline"] = line.pop("roofline_decode_gqa")
    keep = {}
    if dec is not None and not args.no_reference:
        line.update(reference_rows(torch, px, dec, dec_out, ws, stream, args.steps))
        line.update(decode_small_row(torch, px, stream, args.steps, keep=keep))
    if pre is not None and not args.no_reference:
        line.update(prefill_f32_row(torch, px, stream, args.steps, keep=keep))
    if vl is not None:
        vshp = synth.WORKLOADS["prefill_varlen"]
        flops = sum(prefill_flops(1, n, vshp.H, vshp.D) for n in vl["lens"])
        tf = flops / t["prefill_varlen"] / 1e12
        work.append(f"packed causal prefill {vshp.B} sequences ({sum(vl['lens'])} tokens, "
                    f"max {vshp.max_seqlen}) H{vshp.H} D{vshp.D} bf16 "
                    f"({flops / 1e12:.4f} TFLOP/launch)")
        line["prefill_varlen"] = {"ms": t["prefill_varlen"] * 1e3, "tflops": tf,
                                  "frac_mfma_peak": tf / MFMA_BF16_PEAK_TFLOPS,
                                  "flops_per_launch": flops}
        line["roofline_prefill_varlen"] = {
            "bound": "mfma", "achieved": round(tf, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": traffic_for("prefill_varlen", ["fwd_mfma.hip", "pack.hip"]),
            "kernel": "parallax_fwd_varlen call: pack_t_kernel<128,64> + "
                      "fwd_mfma_kernel<D=128, 4 waves> over packed sequences"}
        if dec is None and pre is None and bwd is None and gqa is None:
            line["value"] = round(tf, 2)
            line["unit"] = "TFLOP/s"
            line["roofline"] = line.pop("roofline_prefill_varlen")
    if prj is not None:
        jshp = synth.WORKLOADS["project_qkvr"]
        flops = 2 * jshp.M * jshp.N * jshp.K
        tf = flops / t["project"] / 1e12
        work.append(f"fused qkv+rho projection M{jshp.M} N{jshp.N} K{jshp.K} bf16 "
                    f"({flops / 1e12:.4f} TFLOP/launch)")
        line["project"] = {"ms": t["project"] * 1e3, "tflops": tf,
                           "frac_mfma_peak": tf / MFMA_BF16_PEAK_TFLOPS,
                           "flops_per_launch": flops}
        line["roofline_project"] = {
            "bound": "mfma", "achieved": round(tf, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": traffic_for("project", ["proj.hip"]),
            "kernel": "proj_kernel (256x256 blocks, 16x16x32 bf16 MFMA)"}
        if dec is None and pre is None and bwd is None and gqa is None and vl is None:
            line["value"] = round(tf, 2)
            line["unit"] = "TFLOP/s"
            line["roofline"] = line.pop("roofline_project")
    line["config"]["workload"] = " + ".join(work)
    for n in names:   # per-launch spread of each row's timed launches
        if isinstance(line.get(n), dict):
            line[n].update({k: round(v, 4) for k, v in spread[n].items()})
    if not args.no_cpu_baseline:
        # the oracle on a bounded sample of each row's workload; the first
        # row's goes to cpu_baseline, the others to cpu_baseline_<row>
        base = []
        if dec is not None:
            base.append(("decode", lambda: cpu_baseline_decode(dec, dec_snap)))
        if pre is not None:
            base.append(("prefill", lambda: cpu_baseline_prefill(pre, pre_out)))
        if bwd is not None:
            base.append(("backward", lambda: cpu_baseline_backward(bwd, bwd_dout, bwd_grads)))
        if gqa is not None:
            base.append(("decode_gqa", lambda: cpu_baseline_decode_gqa(gqa, gqa_out)))
        if vl is not None:
            base.append(("prefill_varlen", lambda: cpu_baseline_prefill_varlen(vl, vl["lens"], vl_out)))
        if prj is not None:
            base.append(("project", lambda: cpu_baseline_project(prj, prj_out)))
        if keep.get("decode_small") is not None:
            inp, out = keep["decode_small"]
            base.append(("decode_small", lambda: cpu_baseline_whole_decode(inp, out)))
        if keep.get("prefill_f32") is not None:
            pin, pout = keep["prefill_f32"]
            base.append(("prefill_f32",
                         lambda: cpu_baseline_whole_prefill(pin, pout, tol=1e-4)))
        model = cpu_model()
        for i, (name, fn) in enumerate(base):
            res = fn()
            res["cpu_model"] = model
            res["host_cores"] = cpu_count()
            line["cpu_baseline" if i == 0 else f"cpu_baseline_{name}"] = res
    for key, val in line.items():
        if key.startswith("roofline") and isinstance(val, dict) and "traffic" in val:
            val["traffic_source"] = (
                "copied from profiles/traffic.json (rocprofv3 --pmc FETCH_SIZE, "
                "WRITE_SIZE, copy-calibrated), kept only while the kernel sources "
                "hash to the profiled ones; not measured in this run"
                if val["traffic"] is not None else
                "none: kernel sources changed since the counters were taken")
    print(json.dumps(line), flush=True)


def reference_rows(torch, px, dec, dec_out, ws, stream, steps):
    """Context for the decode row, timed after the step and not part of it:
    the same decode without the probe, and a plain read of the same bytes."""
    import synth
    dshp = synth.WORKLOADS["decode_large"]
    nbytes = decode_bytes(dshp.B, dshp.H, dshp.D, dec["seqlens"].tolist())
    sink = torch.zeros(1, dtype=torch.int32, device=dec["k"].device)
    kv = dec["k"].numel() * dec["k"].element_size() * 2
    fns = [lambda: px.decode(dec["q"], dec["k"], dec["v"], None, dec["seqlens"],
                             out=dec_out, workspace=ws),
           lambda: (px.stream_read(dec["k"], sink), px.stream_read(dec["v"], sink))]
    _, per = time_events(torch, fns, steps, 1, stream, min_warmup_s=0.2)
    soft = nbytes / per[0] / 1e9
    read = kv / per[1] / 1e9
    return {"decode_softmax_only": {"ms": per[0] * 1e3, "gbps": soft,
                                    "frac_hbm_peak": soft / HBM_PEAK_GBPS,
                                    "bytes_per_launch": nbytes},
            "hbm_read_reference": {"ms": per[1] * 1e3, "gbps": read,
                                   "frac_hbm_peak": read / HBM_PEAK_GBPS,
                                   "bytes": kv,
                                   "kernel": "stream_read_kernel, 16-byte non-temporal "
                                             "loads, over the decode K and V"}}


def prefill_f32_row(torch, px, stream, steps, keep=None):
    """The fp32 causal prefill workload (batch 1, 2 heads, seq 256, head_dim
    64: 33.7 MFLOP), timed after the step and not part of it; launches are
    queued behind a GPU spin (a latency-bound point: one fp32 vector-ALU
    decode stream per query row, a few microseconds)."""
    import synth
    shp = synth.WORKLOADS["prefill_f32"]
    dev = torch.device("cuda", 0)
    inp = synth.prefill_inputs(shp, device=dev)
    out = torch.empty((shp.B, shp.N, shp.H, shp.D), device=dev)

    def step():
        px.fwd(inp["q"], inp["k"], inp["v"], inp["rho"], causal=True, out=out)

    n = max(steps, 32)
    t0 = time.perf_counter()
    _, per = time_events(torch, [step], n, 4, stream, min_warmup_s=0.1)
    host_s = (time.perf_counter() - t0) / n
    q = time_queued(torch, step, n, stream, host_s)
    qm = sum(q) / len(q)
    flops = prefill_flops(shp.B, shp.N, shp.H, shp.D)
    if keep is not None:
        step()
        torch.cuda.synchronize()
        keep["prefill_f32"] = (inp, out.clone())
    return {"prefill_f32": {"us": qm * 1e6, "us_median": statistics.median(q) * 1e6,
                            "tflops": flops / qm / 1e12, "flops_per_launch": flops,
                            "us_host_paced": per[0] * 1e6,
                            "kernel": "decode_kernel<fp32, D=64>, one stream per query row "
                                      "(fp32 vector ALU)",
                            "workload": f"causal prefill B{shp.B} N{shp.N} H{shp.H} "
                                        f"D{shp.D} fp32"}}


def decode_small_row(torch, px, stream, steps, nset=16, keep=None):
    """The one-sequence decode workload (batch 1, 16 heads, head_dim 128,
    context 4096: 33.6 MB of K + V), timed after the step and not part of
    it. Launches cycle through `nset` input copies (537 MB at 16) so each
    one streams its K and V from HBM rather than the 256 MB last-level
    cache. At 8 TB/s the bytes take 4.2 us, so this point is bound by launch
    and memory latency."""
    import synth
    shp = synth.WORKLOADS["decode_small"]
    dev = torch.device("cuda", 0)
    one = synth.decode_inputs(shp, device=dev)
    nbytes = decode_bytes(shp.B, shp.H, shp.D, one["seqlens"].tolist())
    sets = [one] + [{k: (t.clone() if k in ("k", "v", "q", "rho") else t)
                     for k, t in one.items()} for _ in range(nset - 1)]
    nspl = px.decode_splits(shp.B, shp.H, shp.D, shp.L)
    wsb = px.decode_workspace_size(shp.B, shp.H, shp.D, shp.L)
    wss = [torch.zeros(max(wsb, 1), dtype=torch.uint8, device=dev) for _ in range(nset)]
    outs = [torch.empty((shp.B, shp.H, shp.D), device=dev) for _ in range(nset)]
    ctr = [0]

    def step():
        i = ctr[0] % nset
        ctr[0] += 1
        st = sets[i]
        px.decode(st["q"], st["k"], st["v"], st["rho"], st["seqlens"], out=outs[i],
                  workspace=wss[i])

    samples = []
    n = max(steps, 4 * nset)
    t0 = time.perf_counter()
    _, per = time_events(torch, [step], n, nset, stream,
                         min_warmup_s=0.2, samples=samples)
    host_s = (time.perf_counter() - t0) / n
    # the same launches enqueued ahead of the GPU (a spin holds the stream
    # while the host queues them): GPU time per call without host gaps
    q = time_queued(torch, step, n, stream, host_s)
    qm = sum(q) / len(q)
    bb = time_back_to_back(torch, step, n, stream, host_s)
    gr = time_graph(torch, step, nset, stream)
    gbps = nbytes / qm / 1e9
    row = {"us": qm * 1e6, "us_min": min(q) * 1e6,
           "us_median": statistics.median(q) * 1e6, "gbps": gbps,
           "frac_hbm_peak": gbps / HBM_PEAK_GBPS, "bytes_per_launch": nbytes,
           "splits": nspl, "input_sets": nset,
           "launches_per_call": 2 if nspl > 1 else 1,
           "timing": "each call bracketed by HIP events on the kernels' stream, "
                     "calls queued behind a GPU spin (no host gaps)",
           "us_back_to_back": bb * 1e6,
           "gbps_back_to_back": nbytes / bb / 1e9,
           "us_graph": gr * 1e6,
           "gbps_graph": nbytes / gr / 1e9,
           "graph_timing": f"one HIP graph holding {nset} calls (one per input set), "
                           "replayed back to back between one pair of events",
           "us_host_paced": per[0] * 1e6,
           "us_host_paced_median": statistics.median(samples[0]) * 1e6,
           "workload": f"decode B{shp.B} H{shp.H} D{shp.D} L{shp.L} bf16"}
    if keep is not None:
        keep["decode_small"] = (one, outs[0].clone())
    del sets, outs, wss
    torch.cuda.empty_cache()
    return {"decode_small": row}


def run_sweep(args):
    """Decode grid: one JSON line per (batch, context, lengths) point."""
    import torch
    import synth
    import transformer_attention_parallax_amd as px

    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream(dev)
    batches = None if args.sweep_batches is None else {int(x) for x in args.sweep_batches.split(",")}
    for B, L in synth.sweep_points():
        if B * L > args.sweep_max_tokens or (batches is not None and B not in batches):
            continue
        for ragged in (False, True):
            shp = synth.DecodeShape(B=B, H=16, D=128, L=L, index=4)
            one = synth.decode_inputs(shp, device=dev, ragged=ragged)
            nbytes = decode_bytes(B, 16, 128, one["seqlens"].tolist())
            # several input sets so that small points stream from HBM, not
            # from the 256 MB last-level cache
            nset = max(1, min(32, math.ceil(1.0e9 / max(nbytes, 1))))
            sets = [one] + [{k: (t.clone() if k in ("k", "v", "q", "rho") else t)
                             for k, t in one.items()} for _ in range(nset - 1)]
            outs = [torch.empty((B, 16, 128), device=dev) for _ in range(nset)]
            wsb = max(16, px.decode_workspace_size(B, 16, 128, L))
            wss = [torch.zeros(wsb, dtype=torch.uint8, device=dev) for _ in range(nset)]
            ctr = [0]

            def step():
                i = ctr[0] % nset
                ctr[0] += 1
                s = sets[i]
                px.decode(s["q"], s["k"], s["v"], s["rho"], s["seqlens"],
                          out=outs[i], workspace=wss[i])
            steps = max(args.steps, 2 * nset)
            t0 = time.perf_counter()
            _, per = time_events(torch, [step], steps, max(args.warmup, nset),
                                 stream)
            host_s = (time.perf_counter() - t0) / steps
            q = time_queued(torch, step, steps, stream, host_s)
            us = sum(q) / len(q)
            gbps = nbytes / us / 1e9
            print(json.dumps({
                "point": {"batch": B, "context": L,
                          "lengths": "ragged" if ragged else "uniform"},
                "us": us * 1e6, "us_host_paced": per[0] * 1e6, "gbps": gbps,
                "frac_hbm_peak": gbps / HBM_PEAK_GBPS,
                "splits": px.decode_splits(B, 16, 128, L),
                "input_sets": nset}), flush=True)
            del sets, one, outs
            torch.cuda.empty_cache()


def run_lla(args):
    """Exact LLA: host conjugate-gradient probe, then one GPU Parallax pass."""
    import numpy as np
    import torch
    import oracle
    import synth
    import transformer_attention_parallax_amd as px

    B, N, H, D = 1, 1024, 4, 128
    shp = synth.PrefillShape(B=B, N=N, H=H, D=D, dtype=torch.float32, index=8)
    inp = synth.prefill_inputs(shp, device="cpu")
    q, k, v = inp["q"], inp["k"], inp["v"]
    threads = cpu_count()
    t0 = time.perf_counter()
    rho, its = oracle.lla_probe(q, k, causal=True, lam=args.lla_lam, threads=threads)
    t_cg = time.perf_counter() - t0
    rho32 = torch.from_numpy(rho).float()
    dev = torch.device("cuda", 0)
    qd, kd, vd, rd = (x.to(dev) for x in (q, k, v, rho32))
    out = torch.empty_like(qd)
    stream = torch.cuda.current_stream(dev)
    fn = lambda: px.fwd(qd, kd, vd, rd, causal=True, out=out)
    _, per = time_events(torch, [fn], args.steps, args.warmup, stream, min_warmup_s=0.2)
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    rows = [(0, int(i), int(h)) for i in rng.integers(0, N, 64) for h in (0, H - 1)]
    ref = oracle.fwd_rows(q, k, v, rho32, rows)
    got = np.stack([out[0, i, h].double().cpu().numpy() for _, i, h in rows])
    n_keys = np.arange(1, N + 1)[None, :, None]
    keys_cg = float(((its + 2) * n_keys).sum())     # softmax + kbar + one pass per CG step
    keys_px = float((n_keys * np.ones_like(its)).sum())
    print(json.dumps({
        "mode": "lla_comparator",
        "workload": f"causal prefill B{B} N{N} H{H} D{D} fp32, seeded N(0,1) q, k, v",
        "lam": args.lla_lam,
        "cg_iterations": {"mean": float(its.mean()), "max": int(its.max())},
        "host_cg_probe_s": t_cg, "host_threads": threads,
        "gpu_parallax_ms": per[0] * 1e3,
        "key_rows_streamed": {"exact_lla_cg": keys_cg, "parallax": keys_px,
                              "ratio": keys_cg / keys_px},
        "max_abs_err_gpu_vs_oracle_lla": float(np.abs(got - ref).max()),
        "sampled_rows": len(rows)}), flush=True)


def run_sweep_gqa(args):
    """Grouped-query decode grid: one JSON line per (batch, context, layout)."""
    import torch
    import synth
    import transformer_attention_parallax_amd as px

    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream(dev)
    G, Hkv, D, P = 4, 8, 128, 16
    Hq = G * Hkv
    points = [(1, 1024), (1, 8192), (1, 32768), (8, 1024), (8, 8192), (8, 32768),
              (64, 2048), (64, 8192), (256, 2048), (256, 8192)]
    for B, L in points:
        for paged in (False, True):
            nbytes = B * L * Hkv * D * 4 + B * Hq * D * 8
            nset = max(1, min(16, math.ceil(1.0e9 / nbytes)))
            sets = []
            for i in range(nset):
                shp = synth.PagedDecodeShape(B=B, Hq=Hq, Hkv=Hkv, D=D, L=L, page=P,
                                             index=10)
                inp = synth.paged_decode_inputs(shp, device=dev, seed_base=10 + i)
                if not paged:   # the same values in a contiguous [B, Hkv, L, D] cache
                    bt = inp["block_table"].long()
                    for name in ("k", "v"):
                        inp[name] = inp[name][bt].reshape(B, L, Hkv, D).transpose(1, 2) \
                            .contiguous()
                    inp["block_table"] = None
                sets.append(inp)
            ns = px.decode_gqa_splits(B, Hq, Hkv, D, L, paged=paged)
            ws = torch.zeros(max(16, px.decode_gqa_workspace_size(B, Hq, Hkv, D, L,
                                                                  paged=paged)),
                             dtype=torch.uint8, device=dev)
            out = torch.empty((B, Hq, D), device=dev)
            ctr = [0]

            def step():
                s = sets[ctr[0] % nset]
                ctr[0] += 1
                px.decode_gqa(s["q"], s["k"], s["v"], s["rho"], seqlens=s["seqlens"],
                              block_table=s["block_table"], out=out, workspace=ws)
            steps = max(args.steps, 2 * nset)
            t0 = time.perf_counter()
            _, per = time_events(torch, [step], steps,
                                 max(args.warmup, nset), stream, min_warmup_s=0.2)
            host_s = (time.perf_counter() - t0) / steps
            q = time_queued(torch, step, steps, stream, host_s)
            us = sum(q) / len(q)
            gbps = nbytes / us / 1e9
            print(json.dumps({"point": {"batch": B, "context": L, "q_heads": Hq,
                                        "kv_heads": Hkv, "paged": paged},
                              "us": us * 1e6, "us_host_paced": per[0] * 1e6,
                              "gbps": gbps,
                              "frac_hbm_peak": gbps / HBM_PEAK_GBPS, "splits": ns,
                              "input_sets": nset}), flush=True)
            del sets
            torch.cuda.empty_cache()


def run_copy_calibration():
    """One device-to-device copy of exactly 1 GiB (reads 1 GiB, writes 1 GiB)."""
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n}), file=sys.stderr, flush=True)
    del src, dst


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU "
              "path (run with --gpus 1).", file=sys.stderr, flush=True)
        sys.exit(2)
    if args.copy_calibration:
        run_copy_calibration()
    elif args.sweep:
        run_sweep(args)
    elif args.lla:
        run_lla(args)
    elif args.sweep_gqa:
        run_sweep_gqa(args)
    else:
        run_main(args)


if __name__ == "__main__":
    main()
