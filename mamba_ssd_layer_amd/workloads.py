"""Seeded synthetic inputs for the SSD forward pass (no method arithmetic here).

This module is shared by the tests, the benchmark and the oracle checks: it
only draws numbers and rounds them to the device dtype.  It computes nothing
of the SSD map itself (no decays, no cumsums, no products), so the oracle and
the HIP path stay independent of each other.

The workloads are Mamba-2-shaped layers: head dim P=64 as in "LLM(十一)——Mamba"
§3.6 (Mamba-2 architecture) and the P in {64, 128} of "Transformers是SSMs…(一)"
§2.4; state sizes N in {16, 128, 256}; B and C shared by all heads of a group
(the grouped multi-input pattern, "LLM(十一)——Mamba" §3.6.2).  The pages name
no speed-benchmark dataset, so every input is synthetic:
  x, B, C ~ N(0, 1) (float32 draws, then rounded to bf16 by round-to-nearest-
  even on the bf16 configs); dt = exp(U(ln lo, ln hi)) per token and head;
  A_head = -exp(U(0, ln 16)) per head.  Draw order: lengths (varlen only),
  x, B, C, u_dt, u_A, all from numpy.random.default_rng(seed).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int            # sequences (batched layout) or packed sequences (varlen)
    seqlen: int           # T per sequence (batched); 0 for varlen
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    chunk_len: int
    dtype: str            # "f32" or "bf16": element type of x, B, C, y
    dt_lo: float = 1e-3
    dt_hi: float = 1e-1
    varlen: bool = False
    len_lo: int = 256     # varlen: lengths ~ U[len_lo, len_hi] (inclusive)
    len_hi: int = 4096
    note: str = ""

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads of the benchmark and parity suite.
WORKLOADS = {
    "tiny_fp32": Workload(
        "tiny_fp32", batch=1, seqlen=256, nheads=1, headdim=64, dstate=16,
        ngroups=1, chunk_len=64, dtype="f32",
        note="batch 1, T=256, H=1, P=64, N=16, G=1, chunk 64, fp32"),
    "mamba2_2p7b_T2k": Workload(
        "mamba2_2p7b_T2k", batch=8, seqlen=2048, nheads=80, headdim=64,
        dstate=128, ngroups=1, chunk_len=256, dtype="bf16",
        note="Mamba-2-2.7B-like layer: batch 8, T=2048, H=80, P=64, N=128, "
             "G=1, chunk 256, bf16"),
    "large_state_T4k": Workload(
        "large_state_T4k", batch=4, seqlen=4096, nheads=32, headdim=64,
        dstate=256, ngroups=1, chunk_len=128, dtype="bf16",
        note="batch 4, T=4096, H=32, P=64, N=256, G=1, chunk 128, bf16"),
    "long_T16k": Workload(
        "long_T16k", batch=1, seqlen=16384, nheads=32, headdim=64,
        dstate=128, ngroups=1, chunk_len=256, dtype="bf16",
        dt_lo=1e-4, dt_hi=1e-2,
        note="batch 1, T=16384, H=32, P=64, N=128, G=1, chunk 256, bf16, "
             "dt ~ exp(U(ln 1e-4, ln 1e-2))"),
    "varlen_16seq": Workload(
        "varlen_16seq", batch=16, seqlen=0, nheads=64, headdim=64,
        dstate=128, ngroups=8, chunk_len=256, dtype="bf16", varlen=True,
        note="16 packed sequences, lengths ~ U[256,4096], H=64, P=64, N=128, "
             "G=8, chunk 256, bf16"),
}


# Decode (one recurrent step per sequence) on a Mamba-2-2.7B-like layer at a
# serving batch: 64 sequences of one token, H=80, P=64, N=128, G=1; x, B, C
# bf16 and the fp32 state.  The pages give no decode configuration; this one
# moves a 168 MB state per step.
DECODE_WORKLOADS = {
    "decode_2p7b_b64": Workload(
        "decode_2p7b_b64", batch=64, seqlen=1, nheads=80, headdim=64, dstate=128,
        ngroups=1, chunk_len=256, dtype="bf16",
        note="decode step: batch 64, H=80, P=64, N=128, G=1, bf16 x/B/C, fp32 state"),
}


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); float32 out.

    Inputs must be finite.  The result holds exactly representable bf16
    values, so a later conversion to a bf16 tensor is exact.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    bias = np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    r = ((u + bias) >> np.uint64(16)) << np.uint64(16)
    return r.astype(np.uint32).view(np.float32).reshape(a.shape)


@dataclass
class Inputs:
    """One seeded input set, in the packed or batched device layout.

    All arrays are numpy.  x, B, C are float32 holding the device values (bf16-
    representable on bf16 workloads).  Batched: x (b,T,H,P), dt (b,T,H),
    B/C (b,T,G,N).  Varlen: x (Ttot,H,P), dt (Ttot,H), B/C (Ttot,G,N) and
    cu_seqlens (S+1,) int32.
    """
    workload: Workload
    x: np.ndarray
    dt: np.ndarray
    A: np.ndarray
    B: np.ndarray
    C: np.ndarray
    cu_seqlens: Optional[np.ndarray] = None
    seqlens: Optional[np.ndarray] = None

    @property
    def total_tokens(self) -> int:
        if self.cu_seqlens is not None:
            return int(self.cu_seqlens[-1])
        return int(self.x.shape[0] * self.x.shape[1])

    def packed_cu_seqlens(self) -> np.ndarray:
        """cu_seqlens of the packed token axis (batched: b equal lengths)."""
        if self.cu_seqlens is not None:
            return self.cu_seqlens.astype(np.int64)
        b, T = self.x.shape[:2]
        return np.arange(b + 1, dtype=np.int64) * T


def make_inputs(w: Workload, seed: int = 0, seqlens=None) -> Inputs:
    """Draw one seeded input set for workload w (see module docstring).

    seqlens: optional explicit list of sequence lengths for a varlen workload
    (then no lengths are drawn; zero lengths are allowed).
    """
    rng = np.random.default_rng(seed)
    H, P, N, G = w.nheads, w.headdim, w.dstate, w.ngroups
    cu = None
    lens = None
    if w.varlen:
        if seqlens is None:
            lens = rng.integers(w.len_lo, w.len_hi + 1, size=w.batch)
        else:
            lens = np.asarray(seqlens, dtype=np.int64)
        cu = np.zeros(len(lens) + 1, dtype=np.int64)
        cu[1:] = np.cumsum(lens)
        lead = (int(cu[-1]),)
    else:
        lead = (w.batch, w.seqlen)
    x = rng.standard_normal(lead + (H, P), dtype=np.float32)
    B = rng.standard_normal(lead + (G, N), dtype=np.float32)
    C = rng.standard_normal(lead + (G, N), dtype=np.float32)
    u_dt = rng.uniform(math.log(w.dt_lo), math.log(w.dt_hi), size=lead + (H,))
    u_A = rng.uniform(0.0, math.log(16.0), size=H)
    dt = np.exp(u_dt).astype(np.float32)
    A = (-np.exp(u_A)).astype(np.float32)
    if w.dtype == "bf16":
        x, B, C = bf16_round(x), bf16_round(B), bf16_round(C)
    elif w.dtype != "f32":
        raise ValueError("dtype must be 'f32' or 'bf16'")
    return Inputs(w, x, dt, A, B, C,
                  None if cu is None else cu.astype(np.int32),
                  None if lens is None else np.asarray(lens, dtype=np.int64))


def initial_states(nseqs: int, nheads: int, headdim: int, dstate: int, seed: int = 0) -> np.ndarray:
    """Seeded initial states (nseqs, nheads, headdim, dstate) float32 ~ N(0, 1),
    from their own generator (default_rng(seed + 1_000_003)) so that drawing
    them leaves the input draws of make_inputs unchanged."""
    rng = np.random.default_rng(seed + 1_000_003)
    return rng.standard_normal((nseqs, nheads, headdim, dstate), dtype=np.float32)


def scan_inputs(batch: int, seqlen: int, channels: int, dstate: int, dtype: str, seed: int = 0):
    """Seeded inputs of the diagonal selective scan (the comparator), drawn like
    the SSD workloads: x, B, C ~ N(0, 1) (rounded to bf16 when dtype is bf16),
    the step size log-uniform in [1e-3, 1e-1] per token and channel, and
    A = -exp(U[0, ln 16]) per (channel, state entry).  Token-major layouts:
    x and delta (batch, seqlen, channels), A (channels, dstate), B and C
    (batch, seqlen, dstate), all float32."""
    rng = np.random.default_rng(seed + 2_000_029)
    x = rng.standard_normal((batch, seqlen, channels), dtype=np.float32)
    B = rng.standard_normal((batch, seqlen, dstate), dtype=np.float32)
    C = rng.standard_normal((batch, seqlen, dstate), dtype=np.float32)
    delta = np.exp(rng.uniform(math.log(1e-3), math.log(1e-1), (batch, seqlen, channels))).astype(np.float32)
    A = (-np.exp(rng.uniform(0.0, math.log(16.0), (channels, dstate)))).astype(np.float32)
    if dtype == "bf16":
        x, B, C = bf16_round(x), bf16_round(B), bf16_round(C)
    return x, delta, A, B, C


def long_device_inputs(seqlen: int, nheads: int, headdim: int, dstate: int, step: float, seed: int, device):
    """Seeded inputs of one very long bf16 sequence, drawn on the device (for a
    tensor too large for host arrays): x, B, C ~ N(0, 1) rounded to bf16 by
    round-to-nearest-even (torch's cast), one B/C group; dt = step * (1 + 0.1 u),
    u ~ U(0, 1) per token and head; A_head = -1.  Draw order from
    torch.Generator(device).manual_seed(seed): x in blocks of 2^18 tokens, B,
    C, u.  Returns device tensors x (1,T,H,P), dt (1,T,H), A (H,), B, C (1,T,1,N)."""
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    x = torch.empty((1, seqlen, nheads, headdim), dtype=torch.bfloat16, device=device)
    blk = 1 << 18
    for t in range(0, seqlen, blk):
        n = min(blk, seqlen - t)
        x[0, t:t + n] = torch.randn((n, nheads, headdim), generator=gen, device=device).to(torch.bfloat16)
    B = torch.randn((1, seqlen, 1, dstate), generator=gen, device=device).to(torch.bfloat16)
    C = torch.randn((1, seqlen, 1, dstate), generator=gen, device=device).to(torch.bfloat16)
    dt = step * (1.0 + 0.1 * torch.rand((1, seqlen, nheads), generator=gen, device=device))
    A = -torch.ones(nheads, dtype=torch.float32, device=device)
    return x, dt.float().contiguous(), A, B, C


def flops_pages(w: Workload, total_tokens: int, seqlens=None) -> dict:
    """FLOP accountings of one forward pass (no arithmetic of the map itself).

    (A) the pages' per-head batched-matmul count ("LLM(十一)——Mamba" §3.5.3):
        per (chunk, head) 2Q^2 N (C B^T) + 2Q^2 P (.X) + 2QNP (chunk states)
        + 2QNP (state -> output) + 2NP (state passing), chunks of Q tokens.
    (B) causal only: Q(Q+1) in place of 2Q^2 in the two diagonal-block terms.
    (C) as (B) with C B^T formed once per group instead of once per head.
    Ragged chunks count their real length.
    """
    H, P, N, G, Q = w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk_len
    if seqlens is None:
        if w.varlen:
            raise ValueError("varlen workload needs its seqlens")
        seqlens = [w.seqlen] * w.batch
    chunks = []
    for L in seqlens:
        L = int(L)
        full, rem = divmod(L, Q)
        chunks += [Q] * full + ([rem] if rem else [])
    a = b = c = 0.0
    for q in chunks:
        a += H * (2 * q * q * N + 2 * q * q * P + 4 * q * N * P + 2 * N * P)
        b += H * (q * (q + 1) * N + q * (q + 1) * P + 4 * q * N * P + 2 * N * P)
        c += G * q * (q + 1) * N + H * (q * (q + 1) * P + 4 * q * N * P + 2 * N * P)
    return {"A_pages": a, "B_causal": b, "C_shared_cbt": c}
