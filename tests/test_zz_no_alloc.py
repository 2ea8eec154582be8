"""The forward entry point that allocates nothing (ssd_chunked_fwd_noalloc:
its workspace is the library's static device scratch) against the
ssd_chunked_fwd entry point it varies, through the C ABI: two calls in a row,
the second smaller, each equal to ssd_chunked_fwd's result bit for bit (the
same kernels on the same inputs) and within the stated bar of the fp64
oracle; a problem past the scratch is refused."""
import numpy as np
import pytest
import torch

from mamba_ssd_layer_amd import _binding as bd
from mamba_ssd_layer_amd.workloads import WORKLOADS, Workload, make_inputs

from gpu_common import TOL, log, max_rel_l2, require_gpu, run_oracle, to_device

pytestmark = pytest.mark.gpu


def _both(inp, dev, Q):
    d = to_device(inp, dev)
    yr, fr = bd.ssd_chunked_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], Q)
    y = torch.full_like(d["x"], float("nan"))
    f = torch.full_like(fr, float("nan"))
    bd.ssd_chunked_fwd_noalloc(d["x"], d["dt"], d["A"], d["B"], d["C"], Q, y, f)
    torch.cuda.synchronize()
    return y, f, yr, fr


def test_noalloc_matches_fwd():
    dev = require_gpu()
    big = make_inputs(WORKLOADS["long_T16k"], 0)
    small = make_inputs(Workload("small", batch=3, seqlen=700, nheads=8, headdim=64, dstate=64,
                                 ngroups=2, chunk_len=128, dtype="bf16"), 1)
    for label, inp in (("long_T16k", big), ("small b=3 T=700 H=8 N=64 Q=128", small)):
        Q = inp.workload.chunk_len
        log(f"[noalloc] {label}")
        y, f, yr, fr = _both(inp, dev, Q)
        assert torch.equal(y, yr), label
        assert torch.equal(f, fr), label
        yo, fo = run_oracle(inp)
        ey, ef = max_rel_l2(y.float().cpu().numpy(), yo, f.cpu().numpy(), fo, inp.packed_cu_seqlens())
        log(f"[noalloc]   max rel-L2 y={ey:.3e} final_state={ef:.3e}")
        assert ey <= TOL[inp.workload.dtype] and ef <= TOL[inp.workload.dtype]


def test_noalloc_refuses_past_its_scratch():
    dev = require_gpu()
    x = torch.empty((1, 65536, 32, 64), dtype=torch.bfloat16, device=dev)
    dt = torch.empty((1, 65536, 32), device=dev)
    A = torch.zeros(32, device=dev)
    B = torch.empty((1, 65536, 1, 128), dtype=torch.bfloat16, device=dev)
    log("[noalloc] past the scratch")
    with pytest.raises(bd.SSDError) as e:
        bd.ssd_chunked_fwd_noalloc(x, dt, A, B, B, 256, torch.empty_like(x))
    assert e.value.status == 5
