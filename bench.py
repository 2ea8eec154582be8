"""Throughput of the SSD forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload long_T16k]

One step = one full forward pass (every kernel: sequence table for varlen
batches, chunk cumsum + chunk states, state passing, chunk output) over one batch of seeded
synthetic inputs already resident in HBM.  The timed region is K steps
bracketed by torch.cuda.synchronize() on both sides; before each step a 512 MiB
read (twice the last-level cache) evicts every cached input, and HIP events on
the launch stream around each step give its time: `value` and `ms_per_step` are
that cold figure (mean; p10/p50/p90 under "timing"), which puts every input
byte on the HBM.  The warm figure (K steps back to back, inputs and
intermediates free to stay in the 256 MiB last-level cache) is reported beside
it, labelled.  A further cold pass of K steps with per-kernel HIP events
(recorded by the library on its launch stream) gives each kernel's average
duration; the roofline of the dominant kernel uses it.  Under "configs" the
other workloads' forward passes are timed the same way (T=2K among them).
The fp64 CPU oracle is timed on the host cores on the same workload (rank 0)
and its output also checks the GPU result.  The line also carries, under
"decode", one recurrent decode step (ssd_decode_step) on 64 sequences of a
Mamba-2-2.7B-like layer (H=80, N=128), with its own HBM roofline
(--no-decode skips it), under "backward" the gradient pass
(ssd_chunked_bwd) on the same workload (--no-backward skips it), and under
"comparator" the diagonal selective scan (ssd_selective_scan, Mamba-1's S6) on
a workload of the same size (one channel per head dimension, the same N and
dtype) with SSD's speed-up over it (--no-comparator skips it), and under
"normalized" the forward with the output divided by its denominator term
(ssd_chunked_fwd_normalized) on the same workload with positive B and C
(--no-normalized skips it), and under "options" the forward with the skip
term D and the dt-scaled input, as a Mamba-2 layer calls it
(ssd_chunked_fwd_ex), on the same workload (--no-options skips it).

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3       # MI355X fp32 matrix
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
METRIC = "SSD fwd tokens/s and TFLOP/s (% bf16 MFMA peak) at T=2K/16K, N=128"
KERNELS = ["seq_table", "chunk_state", "state_pass", "chunk_output"]


def kernel_work(w, seqlens, cb_pass):
    """Algorithmic FLOPs and HBM bytes per launch of each kernel.

    FLOPs follow the pages' batched-matmul count ("LLM(十一)——Mamba" §3.5.3),
    split by the kernel that performs each product, with q the chunk's real
    length: C B^T 2 q^2 N per (chunk, B/C group) (formed once for the heads
    that share B and C: by the kernel-matrix pass when it runs (cb_pass), else
    counted once in chunk_output, which forms the tiles itself), chunk_output
    2 q^2 P + 2 q N P per (chunk, head) ((L o G) X and C h), chunk_state 2 q N P
    per (chunk, head), state_pass 2 N P per (chunk, head).  The headline
    TFLOP/s keeps the pages' per-head count for every term.
    Bytes are each kernel's compulsory reads and writes (e = element bytes,
    Q-padded tables count Q entries per chunk):
      chunk_state  x, B, dt in; states (P N e per chunk-head), Acs (4Q), total (4) out
      chunk_cb     B, C in; causal 32x32 C B^T tiles (e per element) out
      state_pass   states, chunk totals in; passed states out, final state (fp32) out
      chunk_output x, B and C (or C and the C B^T tiles with cb_pass), passed
                   states, Acs in; y out
    """
    H, P, N, G, Q = w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk_len
    e = 2 if w.dtype == "bf16" else 4
    nt = (Q // 32) * (Q // 32 + 1) // 2
    chunks = []
    for L in seqlens:
        full, rem = divmod(int(L), Q)
        chunks += [Q] * full + ([rem] if rem else [])
    T = sum(int(L) for L in seqlens)
    K = len(chunks)
    S = len(seqlens)
    f = {"chunk_state": 0.0, "chunk_cb": 0.0, "state_pass": 0.0, "chunk_output": 0.0}
    for q in chunks:
        f["chunk_cb" if cb_pass else "chunk_output"] += G * 2 * q * q * N
        f["chunk_output"] += H * (2 * q * q * P + 2 * q * N * P)
        f["chunk_state"] += H * 2 * q * N * P
        f["state_pass"] += H * 2 * N * P
    state = K * H * P * N * e
    tiles = K * G * nt * 1024 * e
    b = {
        "chunk_state": T * H * P * e + T * G * N * e + T * H * 4 + state + K * H * (Q + 1) * 4,
        "chunk_cb": (2 * T * G * N * e + tiles) if cb_pass else 0.0,
        "state_pass": state + K * H * 4 + state + S * H * P * N * 4,
        "chunk_output": (T * H * P * e + T * G * N * e * (1 if cb_pass else 2) + state + K * H * Q * 4
                         + (tiles if cb_pass else 0) + T * H * P * e),
    }
    return f, b


def decode_work(w):
    """Algorithmic FLOPs and HBM bytes of one decode step (ssd_decode_step) on
    workload w (batch sequences of one token): per (sequence, head) the fp32
    state is read and written once (8 P N bytes) and 4 P N FLOPs are done
    (2 P N for the update, 2 P N for the output); x, y, dt, B and C are read or
    written once."""
    e = 2 if w.dtype == "bf16" else 4
    b, H, P, N, G = w.batch, w.nheads, w.headdim, w.dstate, w.ngroups
    flops = b * H * 4 * P * N
    byts = b * H * (8 * P * N + 2 * P * e + 4) + H * 4 + 2 * b * G * N * e
    return flops, byts


def bench_decode(bd, torch, steps, warmup, flush):
    """One decode step per sequence on the decode workload: cold (the
    last-level cache flushed before each step, HIP events per step; the
    roofline uses this) and warm (host clock over back-to-back steps), plus the
    kernel's average launch time from the library's HIP events, both ways.
    The fp32 state (168 MB) fits the 256 MiB last-level cache, so only the cold
    figure speaks for HBM."""
    from mamba_ssd_layer_amd.workloads import DECODE_WORKLOADS, initial_states, make_inputs
    w = DECODE_WORKLOADS["decode_2p7b_b64"]
    dev = torch.device("cuda:0")
    inp = make_inputs(w, 0)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    x = torch.from_numpy(inp.x[:, 0]).to(dev).to(tdt).contiguous()
    dt = torch.from_numpy(inp.dt[:, 0]).to(dev).contiguous()
    A = torch.from_numpy(inp.A).to(dev)
    B = torch.from_numpy(inp.B[:, 0]).to(dev).to(tdt).contiguous()
    C = torch.from_numpy(inp.C[:, 0]).to(dev).to(tdt).contiguous()
    state = torch.from_numpy(initial_states(w.batch, w.nheads, w.headdim, w.dstate, 0)).to(dev)
    y = torch.empty_like(x)

    def step():
        bd.ssd_decode_step(x, dt, A, B, C, state, y=y)

    for _ in range(warmup):
        step()
    warm_ms = time_back_to_back(torch, step, steps)
    cold_ev, _ = time_steps(torch, step, steps, flush)
    cold = percentiles(cold_ev)
    kms = kernel_times(bd, torch, step, steps, flush).get("decode_step")
    kms_warm = kernel_times(bd, torch, step, steps).get("decode_step")
    flops, byts = decode_work(w)
    ach = byts / (kms / 1e3) / 1e9 if kms else None
    return {
        "workload": w.name, "batch": w.batch, "nheads": w.nheads, "headdim": w.headdim,
        "dstate": w.dstate, "ngroups": w.ngroups, "dtype": w.dtype,
        "us_per_step": cold["mean"] * 1e3, "tokens_per_s": w.batch / (cold["mean"] / 1e3),
        "cold_ms": cold, "warm_us_per_step": warm_ms * 1e3, "warm_tokens_per_s": w.batch / (warm_ms / 1e3),
        "roofline": {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": ach / PEAK_HBM_GBS if ach else None, "traffic": None,
                     "avg_launch_ms": kms, "avg_launch_ms_warm": kms_warm, "bytes_per_launch": byts,
                     "flops_per_launch": flops,
                     "note": "cold: the state comes from HBM; warm launches partly hit the last-level cache"},
    }


def bench_backward(bd, torch, w, x, dt, A, B, C, cu, steps, warmup):
    """The backward pass (ssd_chunked_bwd) on the forward's workload and inputs,
    with a seeded dy, timed like the forward.  Its roofline counts only the
    compulsory bytes (x, dt, B, C, dy read; dx, d(dt), dB, dC written once):
    the implementation moves several times more (a recompute and three more
    forward-kernel passes on rearranged copies)."""
    import numpy as np
    from mamba_ssd_layer_amd.workloads import bf16_round
    rng = np.random.default_rng(12345)
    dy_np = rng.standard_normal(tuple(x.shape)).astype(np.float32)
    if w.dtype == "bf16":
        dy_np = bf16_round(dy_np)
    dy = torch.from_numpy(dy_np).to(x.device).to(x.dtype)

    def step():
        return bd.ssd_chunked_bwd(x, dt, A, B, C, dy, w.chunk_len, cu_seqlens=cu)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / steps
    e = 2 if w.dtype == "bf16" else 4
    T = int(x.numel() // (w.nheads * w.headdim))
    H, P, N, G = w.nheads, w.headdim, w.dstate, w.ngroups
    byts = 2 * (T * H * P * e + T * H * 4 + 2 * T * G * N * e) + T * H * P * e
    ach = byts / sec / 1e9
    return {"workload": w.name, "us_per_step": sec * 1e6, "tokens_per_s": T / sec,
            "roofline": {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": ach / PEAK_HBM_GBS, "traffic": None, "bytes_per_launch": byts,
                         "note": "compulsory bytes over the whole backward call (several launches)"}}


# v_exp_f32 runs at a quarter of the fp32 lane rate: 256 CUs x 4 SIMDs x 16
# lanes / 4 x 2.4 GHz
PEAK_EXP_GPS = 256 * 4 * 16 / 4 * 2.4


def bench_comparator(bd, torch, w, sec_ssd, steps, warmup):
    """The diagonal selective scan on SSD's workload size: batch and length of
    the workload, D = nheads * headdim channels, the same dstate and dtype.
    Its bound is the exp per (token, channel, state entry) on the vector ALU."""
    import numpy as np
    from mamba_ssd_layer_amd.workloads import scan_inputs
    if w.varlen or w.dstate not in (64, 128, 256):
        return None
    b, T, D, N = w.batch, w.seqlen, w.nheads * w.headdim, w.dstate
    x, delta, A, B, C = scan_inputs(b, T, D, N, w.dtype, 0)
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    xg = torch.from_numpy(np.ascontiguousarray(x.transpose(0, 2, 1))).to(dev).to(tdt)
    dg = torch.from_numpy(np.ascontiguousarray(delta.transpose(0, 2, 1))).to(dev)
    Ag = torch.from_numpy(A).to(dev)
    Bg = torch.from_numpy(B).to(dev).to(tdt)
    Cg = torch.from_numpy(C).to(dev).to(tdt)
    del x, delta, B, C
    y = torch.empty_like(xg)
    for _ in range(warmup):
        bd.ssd_selective_scan(xg, dg, Ag, Bg, Cg, y=y, want_final_state=False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        bd.ssd_selective_scan(xg, dg, Ag, Bg, Cg, y=y, want_final_state=False)
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / steps
    bd.kernel_timing_read(reset=True)
    bd.kernel_timing_enable(True)
    for _ in range(steps):
        bd.ssd_selective_scan(xg, dg, Ag, Bg, Cg, y=y, want_final_state=False)
    torch.cuda.synchronize()
    bd.kernel_timing_enable(False)
    kms = bd.kernel_timing_read(reset=True)["selective_scan"]
    kms = kms[0] / kms[1] if kms[1] else None
    exps = b * T * D * N
    ach = exps / (kms / 1e3) / 1e9 if kms else None
    frac = ach / PEAK_EXP_GPS if ach else None
    # the speed-up at the scan's own bound: what a scan at its exp-rate peak would leave
    bound_sec = exps / (PEAK_EXP_GPS * 1e9)
    return {"kernel": "selective_scan (diagonal A)", "batch": b, "seqlen": T, "channels": D, "dstate": N,
            "dtype": w.dtype, "us_per_step": sec * 1e6, "tokens_per_s": b * T / sec,
            "ssd_speedup": sec / sec_ssd,
            "scan_frac_of_its_bound": frac,
            "ssd_speedup_over_scan_at_its_bound": bound_sec / sec_ssd,
            "note": "both warm; the scan runs below its exp-rate bound, so ssd_speedup overstates the gap "
                    "a scan at its bound would leave (ssd_speedup_over_scan_at_its_bound)",
            "roofline": {"bound": "alu", "achieved": ach, "peak": PEAK_EXP_GPS, "unit": "Gexp/s",
                         "frac": frac, "traffic": None,
                         "avg_launch_ms": kms, "exps_per_launch": exps}}


def time_gpu_back_to_back(torch, step, K):
    """K steps back to back between two HIP events on the current stream (ms
    per step): the GPU's time, whatever the host spends per call."""
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(K):
        step()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / K


def variant_vs_forward(bd, torch, plain, variant, steps, warmup, kernels):
    """A forward variant against the plain forward on the same inputs, both
    warm, outputs preallocated, timed alike (HIP events around back-to-back
    steps, the two alternated three times, each one's best taken); the named
    kernels' launch times of the variant from the library's events."""
    for _ in range(warmup):
        plain()
        variant()
    tp, tv = [], []
    for _ in range(3):
        tp.append(time_gpu_back_to_back(torch, plain, steps))
        tv.append(time_gpu_back_to_back(torch, variant, steps))
    bd.kernel_timing_read(reset=True)
    bd.kernel_timing_enable(True)
    for _ in range(steps):
        variant()
    torch.cuda.synchronize()
    bd.kernel_timing_enable(False)
    kt = bd.kernel_timing_read(reset=True)
    ms_p, ms_v = min(tp), min(tv)
    out = {"us_per_step": ms_v * 1e3, "forward_us_per_step": ms_p * 1e3,
           "overhead_vs_forward": ms_v / ms_p - 1.0}
    for k in kernels:
        out[k + "_us"] = kt[k][0] / kt[k][1] * 1e3 if kt[k][1] else None
    return out


def bench_normalized(bd, torch, w, x, dt, A, B, C, cu, steps, warmup):
    """The normalised forward (y / M 1) on the forward's workload, with B and C
    made positive (|.| + 0.05, the pages' positive feature map), against the
    plain forward on the same inputs, timed alike."""
    Bp = (B.float().abs() + 0.05).to(B.dtype)
    Cp = (C.float().abs() + 0.05).to(C.dtype)
    y = torch.empty_like(x)
    den = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device).reshape(-1, w.nheads)

    def plain():
        if cu is None:
            bd.ssd_chunked_fwd(x, dt, A, Bp, Cp, w.chunk_len, y=y)
        else:
            bd.ssd_chunked_fwd_varlen(x, dt, A, Bp, Cp, cu, w.chunk_len, y=y)

    def variant():
        bd.ssd_chunked_fwd_normalized(x, dt, A, Bp, Cp, w.chunk_len, cu_seqlens=cu, return_final_state=False,
                                      y=y, denom=den)

    r = variant_vs_forward(bd, torch, plain, variant, steps, warmup, ("chunk_output", "chunk_state"))
    r["tokens_per_s"] = int(x.numel() // (w.nheads * w.headdim)) / (r["us_per_step"] * 1e-6)
    r["note"] = ("warm, against the plain forward on the same positive B and C, both timed by HIP events "
                 "around back-to-back steps; the denominator is formed inside the chunk-state "
                 "(ones-column states), state-passing and output kernels")
    return r


def bench_options(bd, torch, w, x, dt, A, B, C, cu, steps, warmup):
    """The forward with the skip term D (one weight per head) and the input
    entering as dt x, on the forward's workload, against the plain forward,
    timed alike."""
    D = torch.linspace(-1.0, 1.0, w.nheads, device=x.device, dtype=torch.float32)
    y = torch.empty_like(x)

    def plain():
        if cu is None:
            bd.ssd_chunked_fwd(x, dt, A, B, C, w.chunk_len, y=y)
        else:
            bd.ssd_chunked_fwd_varlen(x, dt, A, B, C, cu, w.chunk_len, y=y)

    def variant():
        bd.ssd_chunked_fwd_ex(x, dt, A, B, C, w.chunk_len, cu_seqlens=cu, D=D, x_times_dt=True, y=y,
                              return_final_state=False)

    r = variant_vs_forward(bd, torch, plain, variant, steps, warmup, ("chunk_output", "chunk_state"))
    r["options"] = "D and x*dt"
    r["tokens_per_s"] = int(x.numel() // (w.nheads * w.headdim)) / (r["us_per_step"] * 1e-6)
    return r



def min_io_bytes(w, total_tokens, nseq):
    e = 2 if w.dtype == "bf16" else 4
    H, P, N, G = w.nheads, w.headdim, w.dstate, w.ngroups
    return total_tokens * H * (2 * P * e + 4) + 2 * total_tokens * G * N * e + nseq * H * P * N * 4


def load_traffic(kernel, workload):
    """HBM traffic per launch from a committed rocprofv3 counter summary
    (mamba_ssd_layer_amd.prof_summary traffic), used only while the kernel's
    sources still hash to the value the counters were taken on."""
    from mamba_ssd_layer_amd.prof_summary import sources_hash
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    try:
        d = json.load(open(path))
    except (OSError, ValueError):
        return None
    if d.get("sources_sha256_16") != sources_hash(kernel):
        return None
    return d.get("bytes_per_launch")


def load_counters(kernel, workload):
    """Matrix-core utilisation and memory-side request counts of one kernel per
    launch from a committed rocprofv3 counter summary (mamba_ssd_layer_amd.
    prof_summary counters), used only while the kernel's sources still hash to
    the value the counters were taken on; empty otherwise."""
    from mamba_ssd_layer_amd.prof_summary import sources_hash
    path = os.path.join(ROOT, "profiles", f"counters_{kernel}_{workload}.json")
    try:
        d = json.load(open(path))
    except (OSError, ValueError):
        return {"mfma_util": None, "dram_bytes": None}
    if d.get("sources_sha256_16") != sources_hash(kernel):
        return {"mfma_util": None, "dram_bytes": None}
    return {"mfma_util": d.get("mfma_util"), "dram_bytes": d.get("dram_bytes_per_launch"),
            "mfma_flops_counted_per_launch": d.get("mfma_flops_bf16_per_launch")}


class Flusher:
    """Reads a buffer of twice the 256 MiB last-level cache (the Infinity Cache)
    between timed steps, so that each step finds none of its inputs in any
    cache: its reads come from HBM.  Reads leave no dirty lines for the next
    kernel to write back first."""

    def __init__(self, torch, dev, mib=512):
        self.buf = torch.ones((mib << 20) // 4, dtype=torch.float32, device=dev)
        self.out = torch.empty((), dtype=torch.float32, device=dev)
        self.torch = torch

    def __call__(self):
        self.torch.sum(self.buf, dim=0, out=self.out)


def percentiles(ms):
    import numpy as np
    a = np.asarray(ms, dtype=np.float64)
    return {"mean": float(a.mean()), "p10": float(np.percentile(a, 10)), "p50": float(np.percentile(a, 50)),
            "p90": float(np.percentile(a, 90)), "n": int(a.size)}


def time_steps(torch, step, K, flush=None):
    """K steps bracketed by torch.cuda.synchronize() on both sides, each between
    two HIP events on the launch stream (torch's current stream, which the
    binding launches on); with a flush, the cache flush runs before each step's
    first event.  Returns the per-step GPU times (ms) and the host wall time of
    the whole region (s)."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in ev:
        if flush is not None:
            flush()
        a.record()
        step()
        b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return [a.elapsed_time(b) for a, b in ev], wall


def time_back_to_back(torch, step, K):
    """K steps back to back, host clock between two synchronisations (ms per step)."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        step()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / K


def kernel_times(bd, torch, step, K, flush=None):
    """Average launch duration of each library kernel (ms) from the HIP events
    the library records around its launches on the launch stream, over K steps
    (cold when a flush runs before each step)."""
    bd.kernel_timing_read(reset=True)
    bd.kernel_timing_enable(True)
    torch.cuda.synchronize()
    for _ in range(K):
        if flush is not None:
            flush()
        step()
    torch.cuda.synchronize()
    bd.kernel_timing_enable(False)
    kt = bd.kernel_timing_read(reset=True)
    return {k: (v[0] / v[1] if v[1] else None) for k, v in kt.items()}


def forward_setup(bd, torch, w, seed=0):
    """Device inputs of workload w and a step() running one forward pass."""
    import numpy as np
    from mamba_ssd_layer_amd.workloads import make_inputs
    dev = torch.device("cuda:0")
    inp = make_inputs(w, seed)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    t = {"x": torch.from_numpy(inp.x).to(dev).to(tdt), "dt": torch.from_numpy(inp.dt).to(dev),
         "A": torch.from_numpy(inp.A).to(dev), "B": torch.from_numpy(inp.B).to(dev).to(tdt),
         "C": torch.from_numpy(inp.C).to(dev).to(tdt), "cu": None}
    if inp.cu_seqlens is not None:
        t["cu"] = torch.from_numpy(inp.cu_seqlens.astype(np.int32)).to(dev)
        seqlens = np.diff(inp.cu_seqlens).tolist()
    else:
        seqlens = [w.seqlen] * w.batch
    y = torch.empty_like(t["x"])
    fs = torch.empty((len(seqlens), w.nheads, w.headdim, w.dstate), dtype=torch.float32, device=dev)
    x, dt, A, B, C, cu = t["x"], t["dt"], t["A"], t["B"], t["C"], t["cu"]

    def step():
        if cu is None:
            bd.ssd_chunked_fwd(x, dt, A, B, C, w.chunk_len, y=y, final_state=fs)
        else:
            bd.ssd_chunked_fwd_varlen(x, dt, A, B, C, cu, w.chunk_len, y=y, final_state=fs)

    return inp, t, seqlens, y, step


def flop_report(w, tokens, seqlens, sec):
    """TFLOP/s by the executed count (C: causal halves, C B^T once per group,
    what the kernels run) and, labelled, by the pages' per-head count (A)."""
    from mamba_ssd_layer_amd.workloads import flops_pages
    fl = flops_pages(w, tokens, seqlens)
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    c, a = fl["C_shared_cbt"] / sec / 1e12, fl["A_pages"] / sec / 1e12
    return {"executed_C": c, "pct_peak_executed_C": 100.0 * c / peak,
            "pages_A": a, "pct_peak_pages_A": 100.0 * a / peak,
            "causal_B": fl["B_causal"] / sec / 1e12, "peak": peak,
            "note": "C: the products the kernels execute (causal tiles, C B^T once per B/C group); "
                    "A: the per-head batched-matmul count of the pages' cost table (full Q x Q blocks)"}


def config_line(bd, torch, w, K, W, flush):
    """Forward of another workload: cold (cache flushed before each step) and
    warm (back to back) times with percentiles, throughput and FLOP rates, and
    each kernel's cold launch time against its algorithmic bytes."""
    inp, t, seqlens, y, step = forward_setup(bd, torch, w)
    for _ in range(W):
        step()
    cold, _ = time_steps(torch, step, K, flush)
    warm_ms = time_back_to_back(torch, step, K)
    kms = kernel_times(bd, torch, step, K, flush)
    tokens = int(inp.total_tokens)
    c = percentiles(cold)
    sec = c["mean"] / 1e3
    mio = min_io_bytes(w, tokens, len(seqlens))
    kfl, kby = kernel_work(w, seqlens, cb_pass=kms.get("chunk_cb") is not None)
    # per kernel: cold launch time (events) and its algorithmic bytes' share of 8 TB/s
    kern = {k: {"avg_launch_ms": kms[k], "bytes_per_launch": kby[k],
                "hbm_frac": kby[k] / (kms[k] / 1e3) / 1e9 / PEAK_HBM_GBS}
            for k in kby if kby[k] and kms.get(k)}
    del t, y
    return {"workload": w.name, "tokens": tokens, "seqlen": w.seqlen if not w.varlen else None,
            "batch": w.batch, "nheads": w.nheads, "dstate": w.dstate, "ngroups": w.ngroups,
            "chunk_len": w.chunk_len, "dtype": w.dtype,
            "cold_ms": c, "tokens_per_s": tokens / sec, "warm_ms_per_step": warm_ms,
            "warm_tokens_per_s": tokens / (warm_ms / 1e3),
            "tflops": flop_report(w, tokens, seqlens, sec),
            "hbm_min_io": {"bytes": mio, "GBps": mio / sec / 1e9, "pct_peak": 100.0 * mio / sec / 1e9 / PEAK_HBM_GBS},
            "kernels_cold": kern}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # the GPU's clocks take some milliseconds of sustained work to settle; the
    # untimed warmup covers that so the timed steps see the steady state
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--workload", default="long_T16k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the backward-pass measurement reported under \"backward\"")
    ap.add_argument("--no-options", action="store_true",
                    help="skip the forward-with-options measurement reported under \"options\"")
    ap.add_argument("--no-normalized", action="store_true",
                    help="skip the normalised-output measurement reported under \"normalized\"")
    ap.add_argument("--no-comparator", action="store_true",
                    help="skip the selective-scan comparison reported under \"comparator\"")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the decode-step measurement reported under \"decode\"")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workloads' forward lines reported under \"configs\"")
    ap.add_argument("--cold-only", action="store_true",
                    help="time the forward only with the cache flushed (no warm passes): for profiler "
                         "runs whose per-dispatch averages should see cold steps only")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (--steps times), for "
                         "scaling the HBM byte counters of a profiler")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); "
              "the SSD path would shard over (batch, head) with no communication",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.calibrate_copy:
        n = args.calibrate_copy * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_read": n * 4, "calibrate_copy_bytes_written": n * 4,
                          "launches": args.steps}))
        return

    from mamba_ssd_layer_amd import _binding as bd
    from mamba_ssd_layer_amd.workloads import WORKLOADS

    w = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    flush = Flusher(torch, dev)
    inp, t, seqlens, y, step = forward_setup(bd, torch, w)
    x, dt, A, B, C, cu = t["x"], t["dt"], t["A"], t["B"], t["C"], t["cu"]
    nseq = len(seqlens)
    H, P, N = w.nheads, w.headdim, w.dstate
    K = args.steps

    for _ in range(args.warmup):
        step()
    # warm: back to back (every input and intermediate may sit in the caches)
    if args.cold_only:
        warm_ms, warm_ev = float("nan"), [float("nan")]
    else:
        warm_ms = time_back_to_back(torch, step, K)
        warm_ev, _ = time_steps(torch, step, K)
    # cold (the headline): the last-level cache flushed before each step
    cold_ev, cold_wall = time_steps(torch, step, K, flush)
    cold = percentiles(cold_ev)
    ms = cold["mean"]
    # per-kernel durations, cold, from the library's events on its launch stream
    kernel_ms = kernel_times(bd, torch, step, K, flush)
    kernel_ms_warm = {} if args.cold_only else kernel_times(bd, torch, step, K)
    # the output, for the oracle's check below (every step writes the same y)
    y_host = None if args.no_cpu_baseline else y.float().cpu().numpy()

    tokens = int(inp.total_tokens)
    kfl, kby = kernel_work(w, seqlens, cb_pass=kernel_ms.get("chunk_cb") is not None)
    sec = ms / 1e3
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    # per-kernel roofline: the bound is whichever of HBM time and matrix-core
    # time is longer for the kernel's algorithmic bytes and FLOPs
    kroof = {}
    for kname in kfl:
        kms = kernel_ms.get(kname)
        if not kby[kname] and not kfl[kname]:
            continue  # not launched for this configuration
        t_hbm = kby[kname] / (PEAK_HBM_GBS * 1e9)
        t_mfma = kfl[kname] / (peak * 1e12)
        bound = "hbm" if t_hbm >= t_mfma else "mfma"
        if kms:
            ach = (kby[kname] / (kms / 1e3) / 1e9) if bound == "hbm" else (kfl[kname] / (kms / 1e3) / 1e12)
        else:
            ach = None
        pk = PEAK_HBM_GBS if bound == "hbm" else peak
        kroof[kname] = {"bound": bound, "achieved": ach, "peak": pk,
                        "unit": "GB/s" if bound == "hbm" else "TFLOP/s",
                        "frac": (ach / pk) if ach else None, "avg_launch_ms": kms,
                        "avg_launch_ms_warm": kernel_ms_warm.get(kname),
                        "bytes_per_launch": kby[kname], "flops_per_launch": kfl[kname],
                        "tflops_pages_count": kfl[kname] / (kms / 1e3) / 1e12 if kms else None}
    dom = max((k for k in kroof if kroof[k]["avg_launch_ms"]), key=lambda k: kroof[k]["avg_launch_ms"])
    traffic = load_traffic(dom, w.name)
    counters = load_counters(dom, w.name)
    fc = counters.pop("mfma_flops_counted_per_launch", None)
    if fc and kroof[dom]["avg_launch_ms"]:
        # the products the kernel executes (causal tiles), from the matrix-core counters
        counters["mfma_tflops_executed"] = fc / (kroof[dom]["avg_launch_ms"] / 1e3) / 1e12
    mio = min_io_bytes(w, tokens, nseq)

    result = {
        "metric": METRIC,
        "value": tokens / sec,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) x/B/C, log-uniform dt, A=-exp(U(0,ln16)))",
        "config": {"workload": w.name, "batch": w.batch, "seqlen": w.seqlen if not w.varlen else None,
                   "tokens": tokens, "nheads": H, "headdim": P, "dstate": N, "ngroups": w.ngroups,
                   "chunk_len": w.chunk_len, "varlen": w.varlen, "parallelism": "none (1 GPU)"},
        "timing": {"value_from": "cold: mean of per-step HIP-event times, a 512 MiB read flushing the "
                                 "last-level cache before each step (not timed)",
                   "cold_ms": cold, "cold_wall_ms_per_step_with_flush": cold_wall * 1e3 / K,
                   "warm_ms_per_step": warm_ms, "warm_tokens_per_s": tokens / (warm_ms / 1e3),
                   "warm_ms": percentiles(warm_ev)},
        "tflops": flop_report(w, tokens, seqlens, sec),
        "hbm_min_io": {"bytes": mio, "GBps": mio / sec / 1e9,
                       "pct_peak": 100.0 * mio / sec / 1e9 / PEAK_HBM_GBS},
        "kernel_ms": kernel_ms,
        "kernel_ms_warm": kernel_ms_warm,
        "roofline": dict(kroof[dom], kernel=dom, traffic=traffic, **counters),
        "kernel_roofline": kroof,
        "cpu_baseline": None,
    }

    if not args.no_decode:
        result["decode"] = bench_decode(bd, torch, args.steps, min(args.warmup, 200), flush)
    if not args.no_normalized:
        result["normalized"] = bench_normalized(bd, torch, w, x, dt, A, B, C, cu,
                                                min(args.steps, 100), min(args.warmup, 50))
    if not args.no_options:
        result["options"] = bench_options(bd, torch, w, x, dt, A, B, C, cu,
                                          min(args.steps, 100), min(args.warmup, 50))
    if not args.no_comparator:
        result["comparator"] = bench_comparator(bd, torch, w, warm_ms / 1e3, min(args.steps, 20), 3)
    if not args.no_backward:
        result["backward"] = bench_backward(bd, torch, w, x, dt, A, B, C, cu, min(args.steps, 50),
                                            min(args.warmup, 20))

    if not args.no_configs:
        del t, x, dt, A, B, C, y
        result["configs"] = {}
        for name in ("mamba2_2p7b_T2k", "large_state_T4k", "varlen_16seq", "long_T16k"):
            if name == w.name:
                continue
            result["configs"][name] = config_line(bd, torch, WORKLOADS[name], min(K, 100),
                                                  min(args.warmup, 200), flush)
            torch.cuda.empty_cache()

    if not args.no_cpu_baseline:
        import oracle
        cuh = inp.packed_cu_seqlens()
        # bounded sample: the heads of the first sequences, scaled to the workload
        xs = inp.x.reshape(-1, H, P)
        cost = 4.0 * tokens * H * P * N  # oracle FLOPs for the whole workload
        budget = 1.5e11                  # about 10-30 s of fp64 work on a few dozen cores
        hpg = H // w.ngroups             # heads per B/C group: sample whole groups
        hs = H if cost <= budget else max(hpg, int(H * budget / cost) // hpg * hpg)
        gs = hs // hpg
        sel = slice(0, hs)
        def run_oracle():
            return oracle.recurrence(xs[:, sel], inp.dt.reshape(-1, H)[:, sel], inp.A[sel],
                                     inp.B.reshape(-1, w.ngroups, N)[:, :gs],
                                     inp.C.reshape(-1, w.ngroups, N)[:, :gs], cu_seqlens=cuh)
        # repeated until about 10 s of wall time have been measured (at most 100 runs)
        t_o0 = time.perf_counter()
        yo, fo = run_oracle()
        reps = 1
        while time.perf_counter() - t_o0 < 10.0 and reps < 100:
            run_oracle()
            reps += 1
        t_o1 = time.perf_counter()
        scale = H / hs
        o_sec = (t_o1 - t_o0) / reps * scale
        ycpu = y_host.reshape(-1, H, P)[:, sel]
        err = float(np.max(oracle.rel_l2_per_slice(ycpu, yo, slice_axes=(1,))))
        result["cpu_baseline"] = {
            "value": tokens / o_sec, "unit": "tokens/s", "cores": oracle.max_threads(),
            "kind": "oracle",
            "sample": f"fp64 recurrence on {hs} of {H} heads over all {tokens} tokens, "
                      f"{reps} runs in {t_o1 - t_o0:.2f} s wall, scaled x{scale:g} to the workload",
            "gpu_speedup": o_sec / sec,
            "parity_max_rel_l2_y_on_sample": err,
        }
    print(json.dumps(result))


if __name__ == "__main__":
    main()
