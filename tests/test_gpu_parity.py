"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle.

Bar: max relative L2 error over (sequence, head) slices <= 1e-5 for fp32
inputs and <= 2e-2 for bf16 inputs (fp32 accumulation), for y and for the
final state.  Inputs are the seeded synthetic workloads; the oracle reads the
same cast values.  Every case names itself on stdout before it touches the GPU.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from mamba_ssd_layer_amd import _binding as bd
from mamba_ssd_layer_amd.workloads import DECODE_WORKLOADS, WORKLOADS, Workload, initial_states, make_inputs

from gpu_common import TOL, check_parity, log, max_rel_l2, require_gpu, run_gpu, run_oracle, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


# ------------------------------------------------------------ workloads ----
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_tiny_fp32(dev, seed):
    check_parity(make_inputs(WORKLOADS["tiny_fp32"], seed), dev, label=f"tiny_fp32 seed {seed}")


@pytest.mark.parametrize("name", ["mamba2_2p7b_T2k", "large_state_T4k", "long_T16k", "varlen_16seq"])
def test_full_workload_bf16(dev, name):
    """The benchmark workloads at full size, in the launch configuration bench.py times."""
    check_parity(make_inputs(WORKLOADS[name], 0), dev, label=f"{name} full bf16")


@pytest.mark.parametrize("name", ["mamba2_2p7b_T2k", "large_state_T4k", "long_T16k", "varlen_16seq"])
def test_full_shape_fp32(dev, name):
    """The same shapes and chunk lengths with fp32 inputs at 1e-5: a stronger
    check of state passing than bf16 rounding allows."""
    w = WORKLOADS[name].with_(dtype="f32")
    check_parity(make_inputs(w, 0), dev, label=f"{name} full fp32")


# ------------------------------------------------------- shapes / edges ----
SMALL = Workload("small", batch=2, seqlen=300, nheads=4, headdim=64, dstate=64, ngroups=2,
                 chunk_len=64, dtype="bf16")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N", [16, 32, 64, 128, 256])
@pytest.mark.parametrize("Q", [64, 128, 256])
def test_ragged_shapes(dev, dtype, N, Q):
    if not bd.config_supported(torch.bfloat16 if dtype == "bf16" else torch.float32, N, Q):
        pytest.skip("(dtype, N, Q) outside the built set (LDS)")
    w = SMALL.with_(dtype=dtype, dstate=N, chunk_len=Q, seqlen=1000 if Q == 256 else 517)
    check_parity(make_inputs(w, 3), dev, label=f"ragged {dtype} N={N} Q={Q}")


@pytest.mark.parametrize("T", [1, 2, 31, 33, 64, 65, 255, 257])
def test_short_sequences(dev, T):
    for dtype in ("f32", "bf16"):
        w = SMALL.with_(dtype=dtype, seqlen=T, chunk_len=128, batch=3)
        check_parity(make_inputs(w, T), dev, label=f"short T={T} {dtype}")


def test_empty_batch_zero_state(dev):
    log("[edge] seqlen 0")
    w = SMALL.with_(seqlen=0, batch=2)
    inp = make_inputs(w, 0)
    d = to_device(inp, dev)
    y, fs = bd.ssd_chunked_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], 64)
    torch.cuda.synchronize()
    assert y.numel() == 0
    assert torch.all(fs == 0)


def test_chunk_len_invariance(dev):
    """y does not depend on the chunk length beyond rounding (the block
    decomposition is exact for any partition)."""
    w = SMALL.with_(dtype="f32", dstate=64, seqlen=777, batch=2)
    inp = make_inputs(w, 11)
    yr, fr = run_oracle(inp)
    outs = []
    for Q in (64, 128, 256):
        log(f"[invariance] Q={Q}")
        yg, fg = run_gpu(inp, dev, Q)
        ey, ef = max_rel_l2(yg, yr, fg, fr, inp.packed_cu_seqlens())
        assert ey < 1e-5 and ef < 1e-5
        outs.append(yg)
    assert np.max(np.abs(outs[0] - outs[2])) / np.max(np.abs(outs[0])) < 1e-5


def test_varlen_equals_separate_runs(dev):
    """Packed sequences (with empty ones) equal independent batched runs, bit for bit."""
    lens = [300, 0, 1, 513, 64, 0, 77]
    w = SMALL.with_(varlen=True, batch=len(lens), dstate=128, chunk_len=128, nheads=8, ngroups=2)
    inp = make_inputs(w, 21, seqlens=lens)
    log("[varlen] packed run")
    yg, fg = run_gpu(inp, dev)
    cu = inp.packed_cu_seqlens()
    yr, fr = run_oracle(inp)
    ey, ef = max_rel_l2(yg, yr, fg, fr, cu)
    assert ey < 2e-2 and ef < 2e-2
    for s, L in enumerate(lens):
        if L == 0:
            assert np.all(fg[s] == 0)
            continue
        a, b = cu[s], cu[s + 1]
        ws = w.with_(varlen=False, batch=1, seqlen=L)
        from mamba_ssd_layer_amd.workloads import Inputs
        one = Inputs(ws, inp.x[None, a:b], inp.dt[None, a:b], inp.A, inp.B[None, a:b], inp.C[None, a:b])
        log(f"[varlen] sequence {s} alone (L={L})")
        ys, fs = run_gpu(one, dev)
        np.testing.assert_array_equal(ys[0], yg[a:b])
        np.testing.assert_array_equal(fs[0], fg[s])


def test_offsets_beyond_int32(dev):
    """One bf16 sequence of 2^21 + 4173 tokens and 16 heads: x and y hold more
    than 2^31 elements, so every token, head and state offset past that point
    needs 64-bit arithmetic.  Each token decays by about e^-0.2, a chunk of 256
    tokens by more than e^-51 (the whole-chunk mask), so history older than two
    chunks weighs less than e^-100, far below fp32 resolution: y over any window
    equals the oracle run on that window and the two chunks before it from a
    zero state.  Checked at the start, in the middle, past the 2^31-element
    mark and on the ragged last chunk, and likewise the final state."""
    from mamba_ssd_layer_amd.workloads import long_device_inputs
    T, H, P, N, Q = (1 << 21) + 4173, 16, 64, 16, 256
    assert T * H * P > 2 ** 31
    log(f"[int64] drawing {T} tokens x {H} heads on the device")
    x, dt, A, B, C = long_device_inputs(T, H, P, N, 0.2, 11, dev)
    y, fs = bd.ssd_chunked_fwd(x, dt, A, B, C, Q)
    torch.cuda.synchronize()
    An = A.cpu().numpy()
    past = (2 ** 31) // (H * P) + 300  # a token whose x offset is past 2^31 elements
    for t_s in (0, 1 << 20, past, T - 77):
        t_e = min(t_s + Q, T)
        w0 = max(0, t_s - 2 * Q)
        log(f"[int64] window [{t_s}, {t_e}) from {w0}")
        sl = slice(w0, t_e)
        yr, fr = oracle.recurrence(x[0, sl].float().cpu().numpy(), dt[0, sl].cpu().numpy(), An,
                                   B[0, sl].float().cpu().numpy(), C[0, sl].float().cpu().numpy())
        yg = y[0, t_s:t_e].float().cpu().numpy()
        yw = yr[t_s - w0:]
        err = np.linalg.norm(yg - yw, axis=(0, 2)) / np.linalg.norm(yw, axis=(0, 2))
        log(f"[int64]   max rel-L2 over heads {err.max():.3e}")
        assert err.max() < 2e-2
        if t_e == T:
            f = fs[0].cpu().numpy()
            ef = np.linalg.norm((f - fr[0]).reshape(H, -1), axis=1) / np.linalg.norm(fr[0].reshape(H, -1), axis=1)
            log(f"[int64]   final state max rel-L2 {ef.max():.3e}")
            assert ef.max() < 2e-2


def test_forward_repeatable(dev):
    """Every forward entry point gives the same outputs bit for bit on repeated
    calls (no atomics, no order-dependent sums): batched and packed, with the
    skip term, the dt-scaled input and an initial state, and the normalised
    output with its denominator."""
    lens = [700, 0, 257, 1024]
    wb = WORKLOADS["mamba2_2p7b_T2k"].with_(batch=2, seqlen=1024, nheads=16)
    wv = SMALL.with_(varlen=True, batch=len(lens), dstate=128, chunk_len=256, nheads=8, ngroups=2)
    for w, seed, sl in ((wb, 31, None), (wv, 32, lens)):
        inp = make_inputs(w, seed, seqlens=sl)
        d = to_device(inp, dev)
        cu = d.get("cu")
        S = len(lens) if sl else w.batch
        h0 = torch.from_numpy(initial_states(S, w.nheads, w.headdim, w.dstate, seed=seed)).to(dev)
        D = torch.linspace(-1.0, 1.0, w.nheads, device=dev)
        Bp = (d["B"].float().abs() + 0.05).to(d["B"].dtype)
        Cp = (d["C"].float().abs() + 0.05).to(d["C"].dtype)
        calls = {
            "plain": lambda: (bd.ssd_chunked_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], w.chunk_len) if cu is None
                              else bd.ssd_chunked_fwd_varlen(d["x"], d["dt"], d["A"], d["B"], d["C"], cu, w.chunk_len)),
            "options": lambda: bd.ssd_chunked_fwd_ex(d["x"], d["dt"], d["A"], d["B"], d["C"], w.chunk_len, cu_seqlens=cu,
                                                     initial_state=h0, D=D, x_times_dt=True),
            "normalized": lambda: bd.ssd_chunked_fwd_normalized(d["x"], d["dt"], d["A"], Bp, Cp, w.chunk_len,
                                                                cu_seqlens=cu, D=D),
        }
        for name, call in calls.items():
            log(f"[repeat] {w.name} {name}")
            first = [t.clone() for t in call() if t is not None]
            for _ in range(2):
                again = [t for t in call() if t is not None]
                for a1, a2 in zip(first, again):
                    assert torch.equal(a1, a2), name


def test_group_replication(dev):
    """G = H with B, C replicated per head equals G = 1, bit for bit."""
    w = SMALL.with_(ngroups=1, nheads=4, seqlen=400, dstate=128, chunk_len=128)
    inp = make_inputs(w, 5)
    log("[groups] G=1")
    y1, f1 = run_gpu(inp, dev)
    from mamba_ssd_layer_amd.workloads import Inputs
    rep = Inputs(w.with_(ngroups=4), inp.x, inp.dt, inp.A, np.repeat(inp.B, 4, axis=2),
                 np.repeat(inp.C, 4, axis=2))
    log("[groups] G=H replicated")
    y4, f4 = run_gpu(rep, dev)
    np.testing.assert_array_equal(y1, y4)
    np.testing.assert_array_equal(f1, f4)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decay_extremes(dev, dtype):
    """a == 0 (dt*A = -1e4: the oracle gives y_t = (C_t.B_t) x_t) and a == 1
    (A = 0: causal linear attention, no decay at all, so state passing carries
    everything), against the oracle at the dtype's bar."""
    from mamba_ssd_layer_amd.workloads import Inputs
    w = SMALL.with_(dtype=dtype, seqlen=600, dstate=64, chunk_len=128, nheads=2, ngroups=1)
    inp = make_inputs(w, 9)
    z = Inputs(w, inp.x, np.full_like(inp.dt, 1e4), -np.ones_like(inp.A), inp.B, inp.C)
    check_parity(z, dev, label=f"a == 0 {dtype}")
    one = Inputs(w, inp.x * 0.05, inp.dt, np.zeros_like(inp.A), inp.B, inp.C)
    check_parity(one, dev, label=f"a == 1 {dtype}")


def _scaled_decay(inp, ell):
    """The same inputs with A = -4 per head and dt rescaled so that the mean
    dt*A per token is ell."""
    from mamba_ssd_layer_amd.workloads import Inputs
    A = -np.full_like(inp.A, 4.0)
    dt = (inp.dt / inp.dt.mean() * (-ell / 4.0)).astype(np.float32)
    return Inputs(inp.workload, inp.x, dt, A, inp.B, inp.C)


@pytest.mark.parametrize("dtype,Q", [("f32", 128), ("f32", 256), ("bf16", 256), ("bf16", 128)])
@pytest.mark.parametrize("ell", [-0.05, -0.2, -0.5, -1.0, -2.5, -8.0])
def test_large_decays_plain(dev, dtype, Q, ell):
    """The plain forward (ssd_chunked_fwd) with per-token decays from mild to
    extreme: a chunk's total decay of e^(Q ell) selects the whole-chunk mask
    factorisation (within e^16 on fp32, e^64 on bf16), else on bf16 the
    per-tile factorisation when no 32-token tile decays by more than e^64
    (about 32 ell), else the per-element mask, all from one-signed sums
    ("LLM(十一)——Mamba" §3.5.4); each holds the stated bar (dt*A = -8 per
    token: even one 32-token tile decays by e^-256)."""
    w = SMALL.with_(dtype=dtype, dstate=128, chunk_len=Q, seqlen=700, batch=2, nheads=4, ngroups=1)
    check_parity(_scaled_decay(make_inputs(w, 64), ell), dev, label=f"plain {dtype} Q={Q} dt*A~{ell}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_mixed_mask_kinds(dev, dtype):
    """Heads whose decays span the mask factorisations inside one workgroup
    (whole chunk, 32-token tile, per element: A from -0.5 to -40 at dt about
    0.1), so that the output kernel's head loops hand over between kinds, in
    batched and packed form."""
    from mamba_ssd_layer_amd.workloads import Inputs
    w = SMALL.with_(dtype=dtype, dstate=128, chunk_len=256, seqlen=900, batch=2, nheads=8, ngroups=1)
    inp = make_inputs(w, 71)
    A = (-np.exp(np.linspace(np.log(0.5), np.log(40.0), w.nheads))).astype(np.float32)
    dt = (inp.dt / inp.dt.mean() * 0.1).astype(np.float32)
    mixed = Inputs(w, inp.x, dt, A, inp.B, inp.C)
    check_parity(mixed, dev, label=f"mixed kinds {dtype}")
    wv = w.with_(varlen=True, batch=3)
    vin = make_inputs(wv, 72, seqlens=[300, 0, 1100])
    dtv = (vin.dt / vin.dt.mean() * 0.1).astype(np.float32)
    check_parity(Inputs(wv, vin.x, dtv, A, vin.B, vin.C, vin.cu_seqlens), dev, label=f"mixed kinds packed {dtype}")


def test_intermediates_match_chunked_reference(dev):
    """Each kernel on its own: chunk cumsum, chunk states and passed states
    against the oracle's four-step chunked reference."""
    for dtype in ("f32", "bf16"):
        lens = [200, 77, 0, 300]
        w = SMALL.with_(dtype=dtype, varlen=True, batch=len(lens), dstate=32, chunk_len=64,
                        nheads=4, ngroups=2)
        inp = make_inputs(w, 4, seqlens=lens)
        d = to_device(inp, dev)
        log(f"[intermediates] {dtype}")
        out = bd.ssd_chunked_fwd_intermediates(d["x"], d["dt"], d["A"], d["B"], d["C"], 64,
                                               cu_seqlens=d["cu"])
        torch.cuda.synchronize()
        ref = oracle.chunked_steps(inp.x, inp.dt, inp.A, inp.B, inp.C, 64,
                                   cu_seqlens=inp.packed_cu_seqlens())
        K = ref["table"].shape[0]
        acs = out["acs"][:K].cpu().numpy()
        np.testing.assert_allclose(acs, ref["acs"], rtol=1e-5, atol=1e-5)
        tol = 1e-5 if dtype == "f32" else 2e-2
        st = out["states"][:K].cpu().numpy()
        e = oracle.rel_l2_per_slice(st, ref["states"], slice_axes=(0, 1))
        assert np.max(e) < tol, np.max(e)
        hin = out["hin"][:K].cpu().numpy()
        nz = np.array([np.any(ref["hin"][k] != 0) for k in range(K)])
        assert np.all(hin[~nz] == 0)
        e = oracle.rel_l2_per_slice(hin[nz], ref["hin"][nz], slice_axes=(0, 1))
        assert np.max(e) < tol, np.max(e)


# ---------------------------------------------------- head blocks / workspace ----
@pytest.mark.parametrize("dtype,H,G,b,T,Q", [
    ("bf16", 48, 2, 2, 8192, 256),   # 12 heads per workgroup on 256 CUs
    ("bf16", 20, 1, 2, 12800, 256),  # 10
    ("bf16", 64, 1, 2, 16384, 256),  # 32
    ("bf16", 12, 1, 2, 8192, 256),   # 3
    ("f32", 40, 1, 2, 10240, 128),   # 5
    ("bf16", 6, 2, 2, 700, 256),     # 1 (small problem: one head per workgroup)
])
def test_head_block_shapes(dev, dtype, H, G, b, T, Q):
    """Heads per workgroup is any divisor (<= 32) of the heads of a group, chosen
    for the grid's rounds on the device; these shapes give blocks of 12, 10, 32,
    3, 5 and 1 heads on a 256-CU MI355X (the chunk-state prologue scans all of
    a block's heads, one wave per head, several heads per wave above 8)."""
    w = SMALL.with_(dtype=dtype, nheads=H, ngroups=G, batch=b, seqlen=T, dstate=128, chunk_len=Q)
    check_parity(make_inputs(w, 11), dev, label=f"head blocks H={H} G={G} b={b} T={T} Q={Q} {dtype}")


def test_workspace_reuse_across_sizes_and_streams(dev):
    """The workspace is cached per (device, stream) and grown in stream order:
    a small problem, a larger one, the small one again, and the same on a second
    stream, without synchronising in between, all give the results of separate
    synchronised runs (bit for bit: the kernels are deterministic)."""
    small = make_inputs(SMALL.with_(seqlen=400, dstate=128, chunk_len=128), 3)
    large = make_inputs(SMALL.with_(seqlen=3000, nheads=8, dstate=128, chunk_len=256), 4)
    log("[workspace] reference runs")
    ref = {}
    for name, inp in (("small", small), ("large", large)):
        Q = inp.workload.chunk_len
        ref[name] = run_gpu(inp, dev, Q)
    ds = {name: to_device(inp, dev) for name, inp in (("small", small), ("large", large))}
    s2 = torch.cuda.Stream(device=dev)
    s2.wait_stream(torch.cuda.current_stream(dev))  # inputs were made on the current stream
    outs = []
    log("[workspace] interleaved sizes on two streams")
    for stream in (torch.cuda.current_stream(dev), s2):
        with torch.cuda.stream(stream):
            for name in ("small", "large", "small", "large"):
                d = ds[name]
                Q = (small if name == "small" else large).workload.chunk_len
                y, fs = bd.ssd_chunked_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], Q)
                outs.append((name, y, fs))
    torch.cuda.synchronize()
    for name, y, fs in outs:
        yr, fr = ref[name]
        assert np.array_equal(y.float().cpu().numpy(), yr), name
        assert np.array_equal(fs.cpu().numpy(), fr), name


# ------------------------------------------------------- initial state ----
def _oracle_with_init(inp, h0):
    return oracle.recurrence(inp.x, inp.dt, inp.A, inp.B, inp.C, cu_seqlens=inp.packed_cu_seqlens(),
                             init_state=h0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_initial_state_batched(dev, dtype):
    """Batched forward from given initial states against the oracle's recurrence
    started from the same states (the first token's decay now matters)."""
    w = SMALL.with_(dtype=dtype, dstate=128, chunk_len=128, seqlen=700, batch=3, nheads=8, ngroups=2)
    inp = make_inputs(w, 31)
    h0 = initial_states(3, 8, 64, 128, seed=31)
    log(f"[init] batched {dtype} b=3 T=700 H=8 N=128 Q=128")
    d = to_device(inp, dev)
    y, fs = bd.ssd_chunked_fwd_ex(d["x"], d["dt"], d["A"], d["B"], d["C"], 128,
                                  initial_state=torch.from_numpy(h0).to(dev))
    torch.cuda.synchronize()
    yr, fr = _oracle_with_init(inp, h0)
    ey, ef = max_rel_l2(y.float().cpu().numpy(), yr, fs.cpu().numpy(), fr, inp.packed_cu_seqlens())
    log(f"[init]   max rel-L2 y={ey:.3e} final_state={ef:.3e}")
    assert ey <= TOL[dtype] and ef <= TOL[dtype]


def test_initial_state_varlen(dev):
    """Packed sequences (empty ones included) from given initial states; an empty
    sequence's final state is its initial state, exactly."""
    lens = [300, 0, 1, 513, 64, 0, 77]
    w = SMALL.with_(varlen=True, batch=len(lens), dstate=128, chunk_len=128, nheads=8, ngroups=2)
    inp = make_inputs(w, 22, seqlens=lens)
    h0 = initial_states(len(lens), 8, 64, 128, seed=22)
    log("[init] varlen with empty sequences")
    d = to_device(inp, dev)
    y, fs = bd.ssd_chunked_fwd_ex(d["x"], d["dt"], d["A"], d["B"], d["C"], 128, cu_seqlens=d["cu"],
                                  initial_state=torch.from_numpy(h0).to(dev))
    torch.cuda.synchronize()
    fg = fs.cpu().numpy()
    yr, fr = _oracle_with_init(inp, h0)
    ey, ef = max_rel_l2(y.float().cpu().numpy(), yr, fg, fr, inp.packed_cu_seqlens())
    log(f"[init]   max rel-L2 y={ey:.3e} final_state={ef:.3e}")
    assert ey <= TOL["bf16"] and ef <= TOL["bf16"]
    for s, L in enumerate(lens):
        if L == 0:
            np.testing.assert_array_equal(fg[s], h0[s])


def test_ex_without_initial_state_matches_fwd(dev):
    """ssd_chunked_fwd_ex with no initial state is the plain forward, bit for bit,
    in both forms."""
    inp = make_inputs(SMALL.with_(seqlen=600, dstate=128, chunk_len=128), 7)
    d = to_device(inp, dev)
    log("[init] ex(None) vs fwd, batched")
    y0, f0 = bd.ssd_chunked_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], 128)
    y1, f1 = bd.ssd_chunked_fwd_ex(d["x"], d["dt"], d["A"], d["B"], d["C"], 128)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1) and torch.equal(f0, f1)
    lens = [100, 0, 350]
    vin = make_inputs(SMALL.with_(varlen=True, batch=3, dstate=128, chunk_len=128), 8, seqlens=lens)
    dv = to_device(vin, dev)
    log("[init] ex(None) vs fwd, varlen")
    y0, f0 = bd.ssd_chunked_fwd_varlen(dv["x"], dv["dt"], dv["A"], dv["B"], dv["C"], dv["cu"], 128)
    y1, f1 = bd.ssd_chunked_fwd_ex(dv["x"], dv["dt"], dv["A"], dv["B"], dv["C"], 128, cu_seqlens=dv["cu"])
    torch.cuda.synchronize()
    assert torch.equal(y0, y1) and torch.equal(f0, f1)


@pytest.mark.parametrize("name,dtype,Q,T1", [
    ("long_T16k", "bf16", 256, 8192),     # two halves of the long sequence (one GPU's share each)
    ("long_T16k", "bf16", 256, 5000),     # a split inside a chunk
    ("long_T16k", "f32", 128, 6001),
    ("mamba2_2p7b_T2k", "bf16", 256, 1000),
])
def test_split_and_resume(dev, name, dtype, Q, T1):
    """Running tokens [0, T1) and then [T1, T) from the first part's final state
    gives the whole sequence's y and final state: the hand-over of context
    parallelism, each part being one GPU's share at its real shape."""
    w = WORKLOADS[name].with_(dtype=dtype, chunk_len=Q)
    inp = make_inputs(w, 0)
    d = to_device(inp, dev)
    log(f"[split] {name} {dtype} Q={Q} at T1={T1}")
    y1, f1 = bd.ssd_chunked_fwd(*(d[k][:, :T1].contiguous() for k in ("x", "dt")), d["A"],
                                *(d[k][:, :T1].contiguous() for k in ("B", "C")), Q)
    y2, f2 = bd.ssd_chunked_fwd_ex(*(d[k][:, T1:].contiguous() for k in ("x", "dt")), d["A"],
                                   *(d[k][:, T1:].contiguous() for k in ("B", "C")), Q, initial_state=f1)
    torch.cuda.synchronize()
    y = torch.cat([y1, y2], dim=1).float().cpu().numpy()
    yr, fr = run_oracle(inp)
    ey, ef = max_rel_l2(y, yr, f2.cpu().numpy(), fr, inp.packed_cu_seqlens())
    log(f"[split]   max rel-L2 y={ey:.3e} final_state={ef:.3e}")
    assert ey <= TOL[dtype] and ef <= TOL[dtype]


# --------------------------------------------------------- decode step ----
def _slice_rel_l2(got, ref):
    """Max relative L2 over the leading (sequence, head) slices."""
    g = got.reshape(got.shape[0] * got.shape[1], -1).astype(np.float64)
    r = ref.reshape(ref.shape[0] * ref.shape[1], -1).astype(np.float64)
    return float(np.max(np.linalg.norm(g - r, axis=1) / np.maximum(np.linalg.norm(r, axis=1), 1e-300)))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N", [16, 32, 64, 128, 256])
def test_decode_step_vs_oracle(dev, dtype, N):
    """One recurrent step from a random state against the oracle's recurrence
    over one token started from the same state."""
    w = SMALL.with_(dtype=dtype, dstate=N, seqlen=1, batch=5, nheads=8, ngroups=2)
    inp = make_inputs(w, 40 + N)
    h0 = initial_states(5, 8, 64, N, seed=40 + N)
    d = to_device(inp, dev)
    state = torch.from_numpy(h0).to(dev)
    log(f"[decode] {dtype} N={N} batch 5 H=8 G=2")
    y = bd.ssd_decode_step(d["x"][:, 0].contiguous(), d["dt"][:, 0].contiguous(), d["A"],
                           d["B"][:, 0].contiguous(), d["C"][:, 0].contiguous(), state)
    torch.cuda.synchronize()
    yr, fr = oracle.recurrence(inp.x, inp.dt, inp.A, inp.B, inp.C, init_state=h0)
    ey = _slice_rel_l2(y.float().cpu().numpy(), yr[:, 0])
    es = _slice_rel_l2(state.cpu().numpy(), fr)
    log(f"[decode]   max rel-L2 y={ey:.3e} state={es:.3e}")
    assert ey <= TOL[dtype]
    assert es <= 1e-5  # the state stays fp32 on both paths


def test_decode_continues_forward(dev):
    """A forward over tokens [0, T0) and then one decode step per token equals the
    forward over all tokens: y of the decoded tokens and the final state."""
    T0, K = 300, 8
    w = SMALL.with_(dtype="bf16", dstate=128, chunk_len=128, seqlen=T0 + K, batch=3, nheads=8, ngroups=2)
    inp = make_inputs(w, 50)
    d = to_device(inp, dev)
    log(f"[decode] prefill {T0} tokens, then {K} steps")
    _, st = bd.ssd_chunked_fwd(*(d[k][:, :T0].contiguous() for k in ("x", "dt")), d["A"],
                               *(d[k][:, :T0].contiguous() for k in ("B", "C")), 128)
    ys = [bd.ssd_decode_step(*(d[k][:, t].contiguous() for k in ("x", "dt")), d["A"],
                             *(d[k][:, t].contiguous() for k in ("B", "C")), st)
          for t in range(T0, T0 + K)]
    torch.cuda.synchronize()
    yr, fr = run_oracle(inp)
    yd = torch.stack(ys, dim=1).float().cpu().numpy()        # (b, K, H, P)
    ey = _slice_rel_l2(np.moveaxis(yd, 1, 2), np.moveaxis(yr[:, T0:], 1, 2))
    es = _slice_rel_l2(st.cpu().numpy(), fr)
    log(f"[decode]   max rel-L2 y={ey:.3e} state={es:.3e}")
    assert ey <= TOL["bf16"] and es <= TOL["bf16"]


def test_decode_bench_shape(dev):
    """The decode shape bench.py times (64 sequences, H=80, N=128, bf16), every output."""
    w = DECODE_WORKLOADS["decode_2p7b_b64"]
    inp = make_inputs(w, 0)
    h0 = initial_states(w.batch, w.nheads, w.headdim, w.dstate, seed=0)
    d = to_device(inp, dev)
    state = torch.from_numpy(h0).to(dev)
    log("[decode] bench shape")
    y = bd.ssd_decode_step(d["x"][:, 0].contiguous(), d["dt"][:, 0].contiguous(), d["A"],
                           d["B"][:, 0].contiguous(), d["C"][:, 0].contiguous(), state)
    torch.cuda.synchronize()
    yr, fr = oracle.recurrence(inp.x, inp.dt, inp.A, inp.B, inp.C, init_state=h0)
    assert _slice_rel_l2(y.float().cpu().numpy(), yr[:, 0]) <= TOL["bf16"]
    assert _slice_rel_l2(state.cpu().numpy(), fr) <= 1e-5


def test_decode_empty_batch(dev):
    log("[decode] batch 0")
    x = torch.empty((0, 4, 64), dtype=torch.bfloat16, device=dev)
    st = torch.empty((0, 4, 64, 128), dtype=torch.float32, device=dev)
    y = bd.ssd_decode_step(x, torch.empty((0, 4), device=dev), torch.zeros(4, device=dev),
                           torch.empty((0, 1, 128), dtype=torch.bfloat16, device=dev),
                           torch.empty((0, 1, 128), dtype=torch.bfloat16, device=dev), st)
    torch.cuda.synchronize()
    assert y.numel() == 0


# ------------------------------------------- options: skip term, dt input ----
def _run_ex(inp, dev, Q, h0=None, D=None, xdt=False):
    d = to_device(inp, dev)
    kw = dict(initial_state=None if h0 is None else torch.from_numpy(h0).to(dev),
              D=None if D is None else torch.from_numpy(D).to(dev), x_times_dt=xdt)
    if inp.cu_seqlens is not None:
        kw["cu_seqlens"] = d["cu"]
    y, fs = bd.ssd_chunked_fwd_ex(d["x"], d["dt"], d["A"], d["B"], d["C"], Q, **kw)
    torch.cuda.synchronize()
    return y.float().cpu().numpy(), fs.cpu().numpy()


def _check_ex(inp, dev, Q, tol, label, h0=None, D=None, xdt=False):
    log(f"[options] {label}")
    yg, fg = _run_ex(inp, dev, Q, h0, D, xdt)
    assert np.all(np.isfinite(yg)) and np.all(np.isfinite(fg))
    yr, fr = oracle.recurrence(inp.x, inp.dt, inp.A, inp.B, inp.C, cu_seqlens=inp.packed_cu_seqlens(),
                               init_state=h0, D=D, x_times_dt=xdt)
    ey, ef = max_rel_l2(yg, yr, fg, fr, inp.packed_cu_seqlens())
    log(f"[options]   max rel-L2 y={ey:.3e} final_state={ef:.3e}")
    assert ey <= tol and ef <= tol


@pytest.mark.parametrize("dtype,N,Q", [("f32", 64, 128), ("bf16", 128, 256), ("bf16", 256, 64),
                                       ("bf16", 256, 256)])
@pytest.mark.parametrize("D_on,xdt", [(True, False), (False, True), (True, True)])
def test_options_batched(dev, dtype, N, Q, D_on, xdt):
    """The skip term and the dt-scaled input, alone and together, with an initial
    state, against the oracle's recurrence with the same options (bf16 N = Q = 256
    takes the separate kernel-matrix pass)."""
    w = SMALL.with_(dtype=dtype, dstate=N, chunk_len=Q, seqlen=700, batch=2, nheads=8, ngroups=2)
    inp = make_inputs(w, 60 + N)
    h0 = initial_states(2, 8, 64, N, seed=60 + N)
    D = np.random.default_rng(60 + N).standard_normal(8).astype(np.float32)
    _check_ex(inp, dev, Q, TOL[dtype], f"batched {dtype} N={N} Q={Q} D={D_on} x*dt={xdt}",
              h0=h0, D=D if D_on else None, xdt=xdt)


@pytest.mark.parametrize("dtype,N,Q", [("f32", 64, 128), ("bf16", 128, 256)])
def test_options_zero_dt(dev, dtype, N, Q):
    """Tokens with dt = 0, or too small to divide by (1e-30), under the
    dt-scaled input and the skip term: the output kernel's diagonal cannot carry
    D_h x for them through the entry D_h / dt, and the pass after it adds the
    term (every seventh token of every head, a run of 40 tokens of head 1, and
    every eleventh token of head 2 at 1e-30)."""
    from mamba_ssd_layer_amd.workloads import Inputs
    w = SMALL.with_(dtype=dtype, dstate=N, chunk_len=Q, seqlen=600, batch=2, nheads=4, ngroups=1)
    inp = make_inputs(w, 63)
    dt = inp.dt.copy().reshape(2, 600, 4)
    dt[:, 3::7, :] = 0.0
    dt[1, 100:140, 1] = 0.0
    dt[:, 5::11, 2] = 1e-30
    z = Inputs(w, inp.x, dt.reshape(inp.dt.shape), inp.A, inp.B, inp.C)
    D = np.linspace(-1.0, 1.0, 4).astype(np.float32)
    _check_ex(z, dev, Q, TOL[dtype], f"{dtype} N={N} Q={Q} dt = 0 tokens, D and x*dt", D=D, xdt=True)


def test_options_varlen(dev):
    lens = [300, 0, 1, 513, 64, 77]
    w = SMALL.with_(varlen=True, batch=len(lens), dstate=128, chunk_len=128, nheads=8, ngroups=2)
    inp = make_inputs(w, 61, seqlens=lens)
    D = np.random.default_rng(61).standard_normal(8).astype(np.float32)
    _check_ex(inp, dev, 128, TOL["bf16"], "varlen D and x*dt", D=D, xdt=True)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("ell", [-0.05, -0.5, -8.0])
def test_options_large_decays(dev, dtype, ell):
    """The skip term and the dt-scaled input under the whole-chunk mask (dt*A =
    -0.05 per token) and the per-element mask from addition-only segment sums
    (dt*A = -0.5: the chunk decays past e^64; -8: even a 32-token tile does), at
    the stated bar."""
    Q = 256 if dtype == "bf16" else 128
    w = SMALL.with_(dtype=dtype, dstate=64, chunk_len=Q, seqlen=600, batch=2, nheads=4, ngroups=1)
    z = _scaled_decay(make_inputs(w, 62), ell)
    D = np.linspace(-1.0, 1.0, 4).astype(np.float32)
    _check_ex(z, dev, Q, TOL[dtype], f"{dtype} dt*A~{ell} D and x*dt", D=D, xdt=True)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_options(dev, dtype):
    """Decode step with the skip term and the dt-scaled input against the oracle
    over one token from the same state."""
    w = SMALL.with_(dtype=dtype, dstate=128, seqlen=1, batch=6, nheads=8, ngroups=2)
    inp = make_inputs(w, 63)
    h0 = initial_states(6, 8, 64, 128, seed=63)
    D = np.random.default_rng(63).standard_normal(8).astype(np.float32)
    d = to_device(inp, dev)
    state = torch.from_numpy(h0).to(dev)
    log(f"[decode] options {dtype}")
    y = bd.ssd_decode_step(d["x"][:, 0].contiguous(), d["dt"][:, 0].contiguous(), d["A"],
                           d["B"][:, 0].contiguous(), d["C"][:, 0].contiguous(), state,
                           D=torch.from_numpy(D).to(dev), x_times_dt=True)
    torch.cuda.synchronize()
    yr, fr = oracle.recurrence(inp.x, inp.dt, inp.A, inp.B, inp.C, init_state=h0, D=D, x_times_dt=True)
    assert _slice_rel_l2(y.float().cpu().numpy(), yr[:, 0]) <= TOL[dtype]
    assert _slice_rel_l2(state.cpu().numpy(), fr) <= 1e-5


# ------------------------------------------------------------- backward ----
def _grads_gpu(inp, dev, Q, dy, h0=None, D=None, xdt=False, dfinal=None, optional=True):
    d = to_device(inp, dev)
    tdt = torch.bfloat16 if inp.workload.dtype == "bf16" else torch.float32
    tt = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    g = bd.ssd_chunked_bwd(d["x"], d["dt"], d["A"], d["B"], d["C"], tt(dy).to(tdt), Q,
                           cu_seqlens=d.get("cu"), initial_state=tt(h0), D=tt(D), x_times_dt=xdt,
                           dfinal_state=tt(dfinal), want_dD=optional, want_dinitial=optional)
    torch.cuda.synchronize()
    return {k: (None if v is None else v.float().cpu().numpy()) for k, v in g.items()}


def _grad_errors(inp, g, r):
    """Max relative L2 error per (sequence, head) slice for dx and d(dt), per
    (sequence, group) slice for dB and dC, per (sequence, head) for the
    initial-state gradient, and over the head vector for dA and dD."""
    cu = inp.packed_cu_seqlens()
    H, P = inp.x.shape[-2:]
    G, N = inp.B.shape[-2:]

    def per_seq(got, ref):
        """got, ref (Ttot, W, K): max over sequences and W of the relative L2 over (tokens, K)."""
        errs = []
        for s in range(len(cu) - 1):
            a, b = int(cu[s]), int(cu[s + 1])
            if b > a:
                num = np.sqrt(np.sum((got[a:b] - ref[a:b]) ** 2, axis=(0, 2)))
                den = np.sqrt(np.sum(ref[a:b] ** 2, axis=(0, 2)))
                errs.append(num / np.maximum(den, 1e-30))
        return float(np.max(np.concatenate(errs))) if errs else 0.0

    def vec(got, ref):
        return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))

    return {
        "dx": per_seq(g["dx"].reshape(-1, H, P), r["dx"].reshape(-1, H, P)),
        "ddt": per_seq(g["ddt"].reshape(-1, H, 1), r["ddt"].reshape(-1, H, 1)),
        "dB": per_seq(g["dB"].reshape(-1, G, N), r["dB"].reshape(-1, G, N)),
        "dC": per_seq(g["dC"].reshape(-1, G, N), r["dC"].reshape(-1, G, N)),
        "dA": vec(g["dA"], r["dA"]),
        "dD": vec(g["dD"], r["dD"]) if r["dD"] is not None and g["dD"] is not None else 0.0,
        "dinit": (float(np.max(oracle.rel_l2_per_slice(g["dinitial_state"], r["dinit"], slice_axes=(0, 1))))
                  if g["dinitial_state"] is not None else 0.0),
    }


def _check_bwd(inp, dev, Q, tol, label, seed, h0=None, D=None, xdt=False, dfinal=None, optional=True):
    from mamba_ssd_layer_amd.workloads import bf16_round
    rng = np.random.default_rng(seed + 777)
    dy = rng.standard_normal(inp.x.shape).astype(np.float32)
    if inp.workload.dtype == "bf16":
        dy = bf16_round(dy)
    log(f"[bwd] {label}")
    g = _grads_gpu(inp, dev, Q, dy, h0, D, xdt, dfinal, optional)
    for k, v in g.items():
        assert v is None or np.all(np.isfinite(v)), k
    r = oracle.backward(inp.x, inp.dt, inp.A, inp.B, inp.C, dy, cu_seqlens=inp.packed_cu_seqlens(),
                        init_state=h0, dfinal=dfinal, D=D if D is not None else np.zeros(inp.A.shape),
                        x_times_dt=xdt)
    e = _grad_errors(inp, g, r)
    # d(dt) and dA come from d(ell_t) = sum_{k>=t} (dy_k . y_k - x'_k . dx'_k): a
    # running sum of differences whose terms are far larger than the result, so
    # the fp32 recompute's relative error (~5e-7) is magnified by that
    # cancellation (about 20x on these inputs); their fp32 bar is 5e-5
    bars = {k: (max(tol, 5e-5) if k in ("ddt", "dA") else tol) for k in e}
    log("[bwd]   max rel-L2 " + " ".join(f"{k}={v:.2e}" for k, v in e.items()) + f" (bar {tol:g})")
    bad = {k: v for k, v in e.items() if not v <= bars[k]}
    assert not bad, bad


@pytest.mark.parametrize("dtype,N,Q", [("f32", 64, 64), ("f32", 32, 128), ("bf16", 128, 256),
                                       ("bf16", 256, 128), ("bf16", 16, 64)])
def test_backward_batched(dev, dtype, N, Q):
    """Gradients of every input against the oracle's adjoint recurrence, plain
    (no initial state, no dfinal, no options); 520 tokens are not a whole
    number of chunks (bf16 with N >= 64: the padded chunk-local route)."""
    w = SMALL.with_(dtype=dtype, dstate=N, chunk_len=Q, seqlen=520, batch=2, nheads=4, ngroups=2)
    inp = make_inputs(w, 70 + N)
    _check_bwd(inp, dev, Q, TOL[dtype], f"batched {dtype} N={N} Q={Q}", 70 + N)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_all_options(dev, dtype):
    """With an initial state, a final-state gradient, the skip term and the
    dt-scaled input: every gradient, the initial state's included."""
    N, Q = (64, 128) if dtype == "f32" else (128, 256)
    w = SMALL.with_(dtype=dtype, dstate=N, chunk_len=Q, seqlen=700, batch=2, nheads=8, ngroups=2)
    inp = make_inputs(w, 80)
    h0 = initial_states(2, 8, 64, N, seed=80)
    dfin = initial_states(2, 8, 64, N, seed=81)
    D = np.random.default_rng(80).standard_normal(8).astype(np.float32)
    _check_bwd(inp, dev, Q, TOL[dtype], f"options {dtype}", 80, h0=h0, D=D, xdt=True, dfinal=dfin)


@pytest.mark.parametrize("dtype,N,Q,L,opts", [("f32", 64, 64, 512, False), ("bf16", 128, 256, 512, False),
                                                ("bf16", 256, 128, 384, False), ("bf16", 16, 64, 256, False),
                                                ("f32", 64, 128, 512, True), ("bf16", 128, 256, 768, True),
                                                ("bf16", 64, 64, 320, True), ("bf16", 128, 256, 512, "D"),
                                                ("bf16", 128, 256, 512, "xdt")])
def test_backward_chunk_aligned(dev, dtype, N, Q, L, opts):
    """Sequences a whole number of chunks long (the chunk-local d(ell) path),
    plain, with every option, and with the skip term or the dt-scaled input
    alone (dx = dx' unchanged needs neither; dx = dt dx' + D dy otherwise)."""
    w = SMALL.with_(dtype=dtype, dstate=N, chunk_len=Q, seqlen=L, batch=2, nheads=8, ngroups=2)
    seed = 90 + N + L
    inp = make_inputs(w, seed)
    kw = {}
    if opts is True:
        kw = dict(h0=initial_states(2, 8, 64, N, seed=seed), dfinal=initial_states(2, 8, 64, N, seed=seed + 1),
                  D=np.random.default_rng(seed).standard_normal(8).astype(np.float32), xdt=True)
    elif opts == "D":
        D = np.random.default_rng(seed).standard_normal(8).astype(np.float32)
        D[3] = 0.0  # a head whose skip term is zero: dx = dx' there
        kw = dict(D=D)
    elif opts == "xdt":
        kw = dict(xdt=True)
    _check_bwd(inp, dev, Q, TOL[dtype], f"aligned {dtype} N={N} Q={Q} L={L} opts={opts}", seed, **kw)


def test_backward_chunk_aligned_single_subset(dev):
    """Enough chunks x groups x 64-column slices (8 x 16 x 2 x 2 = 512) that
    the per-chunk dB, dC kernel takes each group's heads in one workgroup and
    stores bf16 directly (no partial sums)."""
    w = SMALL.with_(dstate=128, chunk_len=64, seqlen=1024, batch=8, nheads=4, ngroups=2)
    inp = make_inputs(w, 95)
    _check_bwd(inp, dev, 64, TOL["bf16"], "aligned bf16 one head subset", 95, D=np.ones(4, np.float32), xdt=True)


def test_backward_repeatable(dev):
    """The chunk-local bf16 backward gives the same gradients bit for bit on two
    calls: dA is summed per head in chunk order (no atomics), dB and dC from the
    head subsets' partial sums in subset order, the rest per element."""
    from mamba_ssd_layer_amd.workloads import bf16_round
    w = SMALL.with_(dtype="bf16", dstate=128, chunk_len=256, seqlen=2048, batch=2, nheads=8, ngroups=1)
    inp = make_inputs(w, 97)
    dy = bf16_round(np.random.default_rng(97).standard_normal(inp.x.shape).astype(np.float32))
    log("[bwd] repeatable: two calls")
    g1 = _grads_gpu(inp, dev, 256, dy, None, None, True, None, False)
    g2 = _grads_gpu(inp, dev, 256, dy, None, None, True, None, False)
    for k in g1:
        if g1[k] is not None:
            np.testing.assert_array_equal(g1[k], g2[k], err_msg=k)


def test_backward_chunk_aligned_uneven_subsets(dev):
    """64 chunks x 1 group x 2 column slices: the per-chunk dB, dC kernel splits
    the group's 5 heads into subsets of 2 and 3 whose fp32 partial sums are added."""
    w = SMALL.with_(dstate=128, chunk_len=64, seqlen=1024, batch=4, nheads=5, ngroups=1)
    inp = make_inputs(w, 96)
    _check_bwd(inp, dev, 64, TOL["bf16"], "aligned bf16 uneven head subsets", 96)


def test_backward_varlen(dev):
    """Packed sequences, empty ones included (their initial-state gradient is
    dfinal), N = 256 (four 64-column parts)."""
    lens = [300, 0, 1, 513, 64, 0, 77]
    w = SMALL.with_(varlen=True, batch=len(lens), dstate=256, chunk_len=128, nheads=4, ngroups=2)
    inp = make_inputs(w, 82, seqlens=lens)
    h0 = initial_states(len(lens), 4, 64, 256, seed=82)
    dfin = initial_states(len(lens), 4, 64, 256, seed=83)
    _check_bwd(inp, dev, 128, TOL["bf16"], "varlen bf16 N=256", 82, h0=h0, dfinal=dfin)


@pytest.mark.parametrize("optional", [False, True])
def test_backward_varlen_padded(dev, optional):
    """Packed bf16 sequences through the chunk-local path (each sequence padded
    on the device to whole 256-token chunks, an empty sequence among them),
    with and without the optional arrays (initial state, final-state
    gradient, dD and the initial-state gradient)."""
    lens = [700, 0, 45, 1300, 256, 3]
    w = SMALL.with_(varlen=True, batch=len(lens), dstate=128, chunk_len=256, nheads=4, ngroups=2)
    inp = make_inputs(w, 97, seqlens=lens)
    kw = {}
    if optional:
        kw = dict(h0=initial_states(len(lens), 4, 64, 128, seed=97),
                  dfinal=initial_states(len(lens), 4, 64, 128, seed=98),
                  D=np.random.default_rng(97).standard_normal(4).astype(np.float32), xdt=True)
    _check_bwd(inp, dev, 256, TOL["bf16"], f"varlen padded optional={optional}", 97, optional=optional, **kw)


def test_backward_varlen_many_short(dev):
    """Many short packed sequences (padding them to whole chunks would more than
    double the tokens): the role-exchanged passes with fp32 d(ell) instead."""
    lens = [5, 0, 17, 1, 30, 2, 9, 40, 3, 11]
    w = SMALL.with_(varlen=True, batch=len(lens), dstate=64, chunk_len=64, nheads=4, ngroups=2)
    inp = make_inputs(w, 99, seqlens=lens)
    _check_bwd(inp, dev, 64, TOL["bf16"], "varlen many short", 99)


def test_backward_batched_short_fallback(dev):
    """bf16 sequences of 40 tokens with 64-token chunks: too short to pad (the
    padding would more than double them), so the role-exchanged passes with
    fp32 d(ell) run."""
    w = SMALL.with_(dtype="bf16", dstate=64, chunk_len=64, seqlen=40, batch=3, nheads=4, ngroups=2)
    inp = make_inputs(w, 100)
    _check_bwd(inp, dev, 64, TOL["bf16"], "batched short fallback", 100, D=np.ones(4, np.float32), xdt=True)


def test_backward_full_2k(dev):
    """The backward at the Mamba-2-2.7B-like layer's full size (bf16)."""
    inp = make_inputs(WORKLOADS["mamba2_2p7b_T2k"], 0)
    _check_bwd(inp, dev, 256, TOL["bf16"], "mamba2_2p7b_T2k full bf16", 0)


# ------------------------------------------------ selective scan (comparator) ----
def _scan_gpu(dev, x, delta, A, B, C, dtype, offset=0):
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    cv = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    xg = cv(x.transpose(0, 2, 1)).to(tdt)          # channel-major (b, D, T)
    dg = cv(delta.transpose(0, 2, 1))

    def bc(a):  # B or C, starting `offset` elements into its allocation
        t = cv(a).to(tdt)
        if offset == 0:
            return t
        buf = torch.zeros(t.numel() + offset, dtype=tdt, device=dev)
        v = buf[offset:].view(t.shape)
        v.copy_(t)
        return v
    y, fs = bd.ssd_selective_scan(xg, dg, cv(A), bc(B), bc(C))
    torch.cuda.synchronize()
    return y.float().cpu().numpy().transpose(0, 2, 1), fs.cpu().numpy()


def _scan_check(dev, b, T, D, N, dtype, seed, chans=None, offset=0):
    from mamba_ssd_layer_amd.workloads import scan_inputs
    x, delta, A, B, C = scan_inputs(b, T, D, N, dtype, seed)
    log(f"[scan] b={b} T={T} D={D} N={N} {dtype} seed={seed} B/C offset={offset}")
    y, fs = _scan_gpu(dev, x, delta, A, B, C, dtype, offset)
    assert np.all(np.isfinite(y)) and np.all(np.isfinite(fs))
    sel = slice(None) if chans is None else chans   # channels are independent: check a subset
    yr, fr = oracle.selective_scan(x[:, :, sel], delta[:, :, sel], A[sel], B, C)
    tol = TOL[dtype]
    if T > 0:
        ey = float(np.max(oracle.rel_l2_per_slice(y[:, :, sel], yr, slice_axes=(0, 2))))
        assert ey <= tol, ey
    ef = float(np.max(oracle.rel_l2_per_slice(fs[:, sel], fr, slice_axes=(0, 1))))
    assert ef <= tol or (T == 0 and np.all(fs == 0)), ef


@pytest.mark.parametrize("b,T,D,N,dtype", [(2, 200, 6, 64, "f32"), (1, 300, 8, 128, "bf16"),
                                           (3, 65, 5, 256, "f32"), (2, 64, 3, 128, "f32"),
                                           (1, 1, 4, 64, "bf16")])
def test_selective_scan_against_oracle(dev, b, T, D, N, dtype):
    """The comparator against its oracle: blocks of 64 tokens with a ragged
    tail, one to four state entries per lane, a partial last workgroup."""
    _scan_check(dev, b, T, D, N, dtype, 90 + T)


@pytest.mark.parametrize("dtype,N", [("bf16", 128), ("f32", 64), ("bf16", 256)])
def test_selective_scan_unaligned_b_c(dev, dtype, N):
    """B and C one element past a 16-byte boundary (aligned to their element
    only, which the interface allows): the kernel then stages them with
    element loads instead of 16-byte vectors."""
    _scan_check(dev, 2, 150, 9, N, dtype, 95, offset=1)


def test_selective_scan_empty_sequence(dev):
    """T = 0: no output, the final state is the zero initial state."""
    _scan_check(dev, 2, 0, 4, 128, "f32", 91)


def test_selective_scan_full_shape(dev):
    """The comparison shape (one 16384-token sequence, 2048 channels = 32 heads
    of 64, N = 128, bf16), checked on a sample of channels."""
    _scan_check(dev, 1, 16384, 2048, 128, "bf16", 0, chans=np.array([0, 1, 777, 2047]))


# ---------------------------------------------- normalised output (denominator) ----
def _positive(inp):
    """The same inputs with a positive feature map on B and C (|.| + 0.05,
    re-rounded to bf16 on the bf16 path), the pages' condition for positive
    denominators."""
    from mamba_ssd_layer_amd.workloads import bf16_round
    f = (lambda a: bf16_round(np.abs(a) + 0.05)) if inp.workload.dtype == "bf16" else (lambda a: np.abs(a) + 0.05)
    inp.B = f(inp.B).astype(np.float32)
    inp.C = f(inp.C).astype(np.float32)
    return inp


def _check_normalized(inp, dev, Q, label, D=None, xdt=False):
    tol = TOL[inp.workload.dtype]
    d = to_device(inp, dev)
    tt = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    log(f"[norm] {label}")
    y, fs, den = bd.ssd_chunked_fwd_normalized(d["x"], d["dt"], d["A"], d["B"], d["C"], Q,
                                               cu_seqlens=d.get("cu"), D=tt(D), x_times_dt=xdt)
    torch.cuda.synchronize()
    y, fs, den = y.float().cpu().numpy(), fs.cpu().numpy(), den.cpu().numpy()
    yr, fr, dr = oracle.normalized(inp.x, inp.dt, inp.A, inp.B, inp.C,
                                   cu_seqlens=inp.packed_cu_seqlens(), D=D, x_times_dt=xdt)
    H, P = inp.x.shape[-2:]
    cu = inp.packed_cu_seqlens()
    assert np.all(np.isfinite(y)) and np.all(np.isfinite(den))
    ey, ef = max_rel_l2(y.reshape(-1, H, P), yr.reshape(-1, H, P), fs, fr, cu)
    ed = float(np.max(oracle.rel_l2_per_slice(den.reshape(-1, H), dr.reshape(-1, H), slice_axes=(1,))))
    log(f"[norm]   max rel-L2 y {ey:.2e} final_state {ef:.2e} denom {ed:.2e} (bar {tol:g})")
    assert ey <= tol and ef <= tol and ed <= tol


@pytest.mark.parametrize("dtype,N,Q,L", [("f32", 64, 64, 520), ("bf16", 128, 256, 700),
                                         ("bf16", 16, 64, 300), ("f32", 256, 64, 200)])
def test_normalized_batched(dev, dtype, N, Q, L):
    """y / (M 1) against the oracle's extra column of ones: ragged chunks,
    dstate 16..256, several heads per group."""
    w = SMALL.with_(dtype=dtype, dstate=N, chunk_len=Q, seqlen=L, batch=2, nheads=12, ngroups=2)
    inp = _positive(make_inputs(w, 100 + N))
    _check_normalized(inp, dev, Q, f"batched {dtype} N={N} Q={Q} L={L}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_normalized_options(dev, dtype):
    """With the dt-scaled input (the ones column dt-scaled too) and the skip term."""
    w = SMALL.with_(dtype=dtype, dstate=128, chunk_len=128, seqlen=600, batch=2, nheads=8, ngroups=1)
    inp = _positive(make_inputs(w, 110))
    D = np.random.default_rng(110).standard_normal(8).astype(np.float32)
    _check_normalized(inp, dev, 128, f"options {dtype}", D=D, xdt=True)


def test_normalized_varlen(dev):
    """Packed sequences, empty and one-token ones included."""
    lens = [300, 0, 1, 513, 64, 77]
    w = SMALL.with_(dtype="bf16", varlen=True, batch=len(lens), dstate=256, chunk_len=128, nheads=4, ngroups=2)
    inp = _positive(make_inputs(w, 111, seqlens=lens))
    _check_normalized(inp, dev, 128, "varlen bf16 N=256")


def test_normalized_long(dev):
    """4096 tokens x 16 heads, bf16, N = 128, chunk 256 (64 chunks of state passing)."""
    w = SMALL.with_(dtype="bf16", dstate=128, chunk_len=256, seqlen=4096, batch=1, nheads=16, ngroups=1)
    inp = _positive(make_inputs(w, 112))
    _check_normalized(inp, dev, 256, "long bf16")


@pytest.mark.parametrize("dtype,Q", [("f32", 128), ("bf16", 256)])
@pytest.mark.parametrize("ell", [-0.05, -0.5, -8.0])
@pytest.mark.parametrize("opts", [False, True])
def test_normalized_decays(dev, dtype, Q, ell, opts):
    """The denominator under the whole-chunk mask (dt*A = -0.05 per token) and
    the per-element mask (-0.5: the chunk decays past the factorisation's
    limit; -8: every tile does), with and without the skip term and the
    dt-scaled input; 16 heads (two workgroups' head blocks of the normalised
    output)."""
    w = SMALL.with_(dtype=dtype, dstate=64, chunk_len=Q, seqlen=700, batch=2, nheads=16, ngroups=2)
    inp = _positive(_scaled_decay(make_inputs(w, 113), ell))
    D = np.linspace(-1.0, 1.0, 16).astype(np.float32) if opts else None
    _check_normalized(inp, dev, Q, f"{dtype} Q={Q} dt*A~{ell} options={opts}", D=D, xdt=opts)
