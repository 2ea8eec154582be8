"""Helpers of the GPU parity tests: move seeded inputs to the device, run the
HIP path through the C ABI, run the fp64 oracle on the same cast values, and
compare with the max relative L2 error over (sequence, head) slices."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from mamba_ssd_layer_amd import _binding as bd
from mamba_ssd_layer_amd.workloads import Inputs

TOL = {"f32": 1e-5, "bf16": 2e-2}


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def require_gpu():
    assert torch.cuda.is_available(), "GPU test run without a GPU"
    return torch.device("cuda:0")


def to_device(inp: Inputs, dev):
    tdt = torch.bfloat16 if inp.workload.dtype == "bf16" else torch.float32
    d = dict(
        x=torch.from_numpy(inp.x).to(dev).to(tdt).contiguous(),
        dt=torch.from_numpy(inp.dt).to(dev).contiguous(),
        A=torch.from_numpy(inp.A).to(dev).contiguous(),
        B=torch.from_numpy(inp.B).to(dev).to(tdt).contiguous(),
        C=torch.from_numpy(inp.C).to(dev).to(tdt).contiguous(),
    )
    if inp.cu_seqlens is not None:
        d["cu"] = torch.from_numpy(inp.cu_seqlens.astype(np.int32)).to(dev)
    return d


def run_gpu(inp: Inputs, dev, chunk_len=None):
    Q = chunk_len or inp.workload.chunk_len
    d = to_device(inp, dev)
    if inp.cu_seqlens is not None:
        y, fs = bd.ssd_chunked_fwd_varlen(d["x"], d["dt"], d["A"], d["B"], d["C"], d["cu"], Q)
    else:
        y, fs = bd.ssd_chunked_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], Q)
    torch.cuda.synchronize()
    return y.float().cpu().numpy(), fs.cpu().numpy()


def run_oracle(inp: Inputs):
    cu = inp.packed_cu_seqlens()
    return oracle.recurrence(inp.x, inp.dt, inp.A, inp.B, inp.C, cu_seqlens=cu)


def max_rel_l2(y_got, y_ref, fs_got, fs_ref, cu):
    """Max relative L2 over (sequence, head) slices of y and of final_state."""
    H, P = y_ref.shape[-2:]
    yg = y_got.reshape(-1, H, P)
    yr = y_ref.reshape(-1, H, P)
    ey = []
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        if b > a:
            ey.append(oracle.rel_l2_per_slice(yg[a:b], yr[a:b], slice_axes=(1,)))
    ey = np.concatenate(ey) if ey else np.zeros(1)
    ef = oracle.rel_l2_per_slice(fs_got, fs_ref, slice_axes=(0, 1))
    return float(np.max(ey)), float(np.max(ef))


def check_parity(inp: Inputs, dev, chunk_len=None, tol=None, label=""):
    tol = tol if tol is not None else TOL[inp.workload.dtype]
    log(f"[parity] {label or inp.workload.name} Q={chunk_len or inp.workload.chunk_len} "
        f"tokens={inp.total_tokens}")
    yg, fg = run_gpu(inp, dev, chunk_len)
    assert np.all(np.isfinite(yg)) and np.all(np.isfinite(fg)), "non-finite output"
    yr, fr = run_oracle(inp)
    ey, ef = max_rel_l2(yg, yr, fg, fr, inp.packed_cu_seqlens())
    log(f"[parity]   max rel-L2 y={ey:.3e} final_state={ef:.3e} (tol {tol:g})")
    assert ey <= tol, f"y rel-L2 {ey} > {tol}"
    assert ef <= tol, f"final_state rel-L2 {ef} > {tol}"
    return ey, ef
