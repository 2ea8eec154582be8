"""fp64 CPU oracle of the SSD (state space duality) layer forward pass.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  It
shares no code with the HIP path (``mamba_ssd_layer_amd``) and imports nothing
from it; the two meet only at the seeded input generators, which hold none of
the method's arithmetic.

Pages cited (titles as published):
  [T] "Transformers是SSMs：通过结构化状态空间对偶性的广义模型和高效算法(一)"
      (nxbn.cn/automobile/1783.html), sections 1-5 of "Transformers are SSMs".
  [M] "LLM(十一)——Mamba" (mztchaoqun.com.cn/posts/D49_Mamba).
  [S] "Mamba-2 状态空间对偶性理论" (metaphor-xennon.pages.dev).

The map, its forms and its gradients, all fp64:
  recurrence()     O1, the oracle of record: the plain recurrence of [T] §2.4 /
                   §5.1 and [M] §3.1.2, in C (ssd_oracle.c) with OpenMP over
                   (sequence, head).
  backward()       O4, the gradients of O1 (the adjoint recurrence, in C):
                   the training direction the pages price but do not derive
                   ([M] §3.5.3 cost table; pinned by finite differences).
  quadratic()      O2, the dual form Y = (L o C B^T) X of [T] §2.4 and [M]
                   §3.1.3 with L the 1-semiseparable matrix of [T] §3.2.2, by
                   brute force; tiny inputs only.
  normalized()     O6, the output divided by its denominator term M 1 (one
                   more column of ones on X), [T]/[M] normalisation term.
  selective_scan() O5, the comparator: the selective scan with a diagonal
                   transition of Mamba-1 ([M] §3.1.1-3.1.2, §2.1.2-2.1.3), in C.
  chunked_steps()  O3, the four steps of the block decomposition of [M] §3.5
                   ("SSD algorithm: chunking and state passing"), exposing the
                   per-chunk log-decay cumsum, chunk states and passed states
                   so that a GPU kernel's intermediate can be checked alone.
Every function here is pinned by tests/test_oracle.py against closed forms,
brute force and invariants that do not reuse its own code.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssd_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libssd_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile ssd_oracle.c with gcc (-O2, OpenMP) into libssd_oracle.so."""
    global _lib
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
        _lib = None
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or (
                os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        i64p = ctypes.POINTER(ctypes.c_int64)
        lib.ssd_oracle_recurrence.argtypes = [
            dp, dp, dp, dp, dp, i64p, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, dp, dp, dp,
            ctypes.c_int]
        lib.ssd_oracle_recurrence.restype = ctypes.c_int
        lib.ssd_oracle_backward.argtypes = [
            dp, dp, dp, dp, dp, i64p, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, dp, dp, dp, dp, dp,
            dp, dp, dp, dp, ctypes.c_int]
        lib.ssd_oracle_backward.restype = ctypes.c_int
        lib.ssd_oracle_selective_scan.argtypes = [
            dp, dp, dp, dp, dp, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_int64, dp, dp, ctypes.c_int]
        lib.ssd_oracle_selective_scan.restype = ctypes.c_int
        lib.ssd_oracle_max_threads.argtypes = []
        lib.ssd_oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def max_threads() -> int:
    """Threads an OpenMP region of the oracle uses by default."""
    return int(_load().ssd_oracle_max_threads())


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a, ctype=ctypes.c_double):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def recurrence(x, dt, A, B, C, cu_seqlens=None, init_state=None, nthreads=0, D=None,
               x_times_dt=False):
    """O1: fp64 naive recurrence ([T] §2.4, §3.1 eq. (3), §5.1; [M] §3.1.2).

    Packed layout: x (Ttot,H,P), dt (Ttot,H), A (H,), B and C (Ttot,G,N),
    cu_seqlens (S+1,) with cu[0]=0 and cu[S]=Ttot (None: one sequence).
    A batched input (b,T,...) may be passed; it is treated as b sequences of
    length T.  init_state (S,H,P,N) or None (zero).
    Options of the layer around the recurrence:
      x_times_dt  the input enters the state as dt_t x_t (B scaled by the step
                  size: the first-order discretisation Mamba-2 keeps from
                  Mamba, [M] "离散化" after §3.5.4; the pages print no formula,
                  so this reading is a convention: parity unpinned by the
                  pages, pinned by the closed form in the tests);
      D (H,)      skip term y_t += D_h x_t on the raw input ([M] §1.2: D
                  passes the input straight to the output).
    Returns y with x's leading shape and final_state (S,H,P,N), both fp64.
    """
    x = _f64(x)
    x_raw = x
    if x_times_dt:
        x = x * _f64(dt)[..., None]
    lead = x.shape[:-2]
    H, P = x.shape[-2:]
    if x.ndim == 4:  # (b, T, H, P) batched
        b, T = x.shape[:2]
        if cu_seqlens is None:
            cu_seqlens = np.arange(b + 1, dtype=np.int64) * T
    Ttot = int(np.prod(lead))
    x = x.reshape(Ttot, H, P)
    dt = _f64(dt).reshape(Ttot, H)
    A = _f64(A).reshape(H)
    N = B.shape[-1]
    G = B.shape[-2]
    B = _f64(B).reshape(Ttot, G, N)
    C = _f64(C).reshape(Ttot, G, N)
    if cu_seqlens is None:
        cu_seqlens = np.array([0, Ttot], dtype=np.int64)
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    S = cu.shape[0] - 1
    if cu[-1] != Ttot:
        raise ValueError("cu_seqlens[-1] must equal the packed length")
    y = np.empty((Ttot, H, P), dtype=np.float64)
    fs = np.empty((S, H, P, N), dtype=np.float64)
    init = None
    if init_state is not None:
        init = _f64(init_state).reshape(S, H, P, N)
    rc = _load().ssd_oracle_recurrence(
        _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C),
        _ptr(cu, ctypes.c_int64), S, H, P, N, G,
        _ptr(init) if init is not None else None, _ptr(y), _ptr(fs),
        int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    y = y.reshape(*lead, H, P)
    if D is not None:
        y = y + _f64(D).reshape(H)[:, None] * x_raw.reshape(*lead, H, P)
    return y, fs


def backward(x, dt, A, B, C, dy, cu_seqlens=None, init_state=None, dfinal=None, D=None,
             x_times_dt=False, nthreads=0):
    """O4: fp64 backward of O1 with its options: the gradients of a loss L with
    dL/dy = dy and dL/d(final state) = dfinal (None: 0), by the adjoint
    recurrence of ssd_oracle.c (the chain rule through h_t = a_t h_{t-1} +
    x_t B_t^T, y_t = h_t C_t in reverse token order).  With x_times_dt the
    recurrence sees x' = dt x, so dx = dt dx' and d(dt) gains x . dx'; with D,
    y += D x adds D dy to dx and gives dD = sum_t x_t . dy_t.
    Layouts as recurrence().  Returns a dict of fp64 arrays: dx (x's shape),
    ddt (dt's shape), dA (H,), dB and dC (B's shape, summed over each group's
    heads), dD (H,) or None, dinit (S,H,P,N).
    """
    x = _f64(x)
    lead = x.shape[:-2]
    H, P = x.shape[-2:]
    if x.ndim == 4 and cu_seqlens is None:
        b, T = x.shape[:2]
        cu_seqlens = np.arange(b + 1, dtype=np.int64) * T
    Ttot = int(np.prod(lead))
    x = x.reshape(Ttot, H, P)
    dtv = _f64(dt).reshape(Ttot, H)
    A = _f64(A).reshape(H)
    N = B.shape[-1]
    G = B.shape[-2]
    Bv = _f64(B).reshape(Ttot, G, N)
    Cv = _f64(C).reshape(Ttot, G, N)
    dyv = _f64(dy).reshape(Ttot, H, P)
    if cu_seqlens is None:
        cu_seqlens = np.array([0, Ttot], dtype=np.int64)
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    S = cu.shape[0] - 1
    xin = x * dtv[:, :, None] if x_times_dt else x
    init = None if init_state is None else _f64(init_state).reshape(S, H, P, N)
    dfin = None if dfinal is None else _f64(dfinal).reshape(S, H, P, N)
    dxp = np.empty((Ttot, H, P))
    ddt = np.empty((Ttot, H))
    dA = np.empty((S, H))
    dBh = np.empty((Ttot, H, N))
    dCh = np.empty((Ttot, H, N))
    dinit = np.empty((S, H, P, N))
    rc = _load().ssd_oracle_backward(
        _ptr(xin), _ptr(dtv), _ptr(A), _ptr(Bv), _ptr(Cv), _ptr(cu, ctypes.c_int64), S, H, P, N, G,
        _ptr(init) if init is not None else None, _ptr(dyv), _ptr(dfin) if dfin is not None else None,
        _ptr(dxp), _ptr(ddt), _ptr(dA), _ptr(dBh), _ptr(dCh), _ptr(dinit), int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    dx = dxp
    if x_times_dt:
        ddt = ddt + np.einsum("thp,thp->th", x, dxp)
        dx = dxp * dtv[:, :, None]
    dD = None
    if D is not None:
        dx = dx + _f64(D).reshape(H)[None, :, None] * dyv
        dD = np.einsum("thp,thp->h", x, dyv)
    hpg = H // G
    dB = dBh.reshape(Ttot, G, hpg, N).sum(axis=2)
    dC = dCh.reshape(Ttot, G, hpg, N).sum(axis=2)
    return dict(dx=dx.reshape(*lead, H, P), ddt=ddt.reshape(np.shape(dt)), dA=dA.sum(axis=0),
                dB=dB.reshape(np.shape(B)), dC=dC.reshape(np.shape(C)), dD=dD, dinit=dinit)


def normalized(x, dt, A, B, C, cu_seqlens=None, D=None, x_times_dt=False, nthreads=0):
    """O6: the SSD output normalised by its denominator term ([T]/[M]
    "Incorporating a Normalization (Denominator) Term", next to the kernel
    feature maps): the denominator of Y = M X is M 1, found by giving X one
    more column of ones, (T, P) -> (T, P + 1); the output is the first P
    columns divided by the last.  The extra column enters the state like x (so
    it is dt-scaled with the dt-scaled input) from a zero state; the skip term
    D x is added after the division.  The pages require a positive feature
    map so that the denominators are positive; callers pass such B and C.

    Layout as recurrence().  Returns (y, final_state, denom) with final_state
    (S, H, P, N) the state of the P columns of x and denom (Ttot, H)."""
    x = _f64(x)
    lead = x.shape[:-2]
    H, P = x.shape[-2:]
    ones = np.ones(lead + (H, 1))
    xe = np.concatenate([x, ones], axis=-1)
    ye, fse = recurrence(xe, dt, A, B, C, cu_seqlens=cu_seqlens, nthreads=nthreads,
                         x_times_dt=x_times_dt)
    denom = ye[..., P]
    y = ye[..., :P] / denom[..., None]
    if D is not None:
        y = y + _f64(D).reshape(H)[:, None] * x
    return y, fse[..., :P, :], denom.reshape(-1, H)


def selective_scan(x, delta, A, B, C, nthreads=0):
    """O5: fp64 selective scan with a diagonal transition (Mamba-1's S6), the
    comparator of the SSD layer ([M] §3.1.1-3.1.2: a diagonal A, of which SSD
    keeps one scalar; §2.1.2-2.1.3: one SSM per channel, Delta per token and
    channel, B and C per token).  h_t = exp(Delta_t A) o h_{t-1} + Delta_t x_t B_t
    per channel (state N), y_t = C_t . h_t, zero state per sequence.

    x, delta (b, T, D); A (D, N); B, C (b, T, N).  Returns y (b, T, D) and the
    final state (b, D, N), fp64.
    """
    x = _f64(x)
    nb, T, D = x.shape
    N = A.shape[-1]
    delta = _f64(delta).reshape(nb, T, D)
    A = _f64(A).reshape(D, N)
    B = _f64(B).reshape(nb, T, N)
    C = _f64(C).reshape(nb, T, N)
    y = np.empty((nb, T, D), dtype=np.float64)
    fs = np.empty((nb, D, N), dtype=np.float64)
    rc = _load().ssd_oracle_selective_scan(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C),
                                           nb, T, D, N, _ptr(y), _ptr(fs), int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return y, fs


def quadratic(x, dt, A, B, C):
    """O2: brute-force dual form for ONE sequence (tiny T only).

    [T] §3.1 eq. (3): M[j, i] = C_j^T (a_j ... a_{i+1}) B_i for j >= i, else 0;
    [T] §2.4 / [M] §3.1.3: M = L o (C B^T) with L = 1SS(a) of [T] §3.2.2
    (the empty product on the diagonal is 1).  Y = M X per head.
    Shapes: x (T,H,P), dt (T,H), A (H,), B and C (T,G,N).  Returns y (T,H,P).
    """
    x = _f64(x)
    T, H, P = x.shape
    G = B.shape[1]
    a = np.exp(_f64(dt) * _f64(A)[None, :])  # (T, H)
    B = _f64(B)
    C = _f64(C)
    y = np.zeros_like(x)
    for h in range(H):
        g = h * G // H
        L = np.zeros((T, T))
        for j in range(T):
            prod = 1.0
            L[j, j] = 1.0
            for i in range(j - 1, -1, -1):
                prod *= a[i + 1, h]
                L[j, i] = prod
        M = L * (C[:, g, :] @ B[:, g, :].T)
        y[:, h, :] = M @ x[:, h, :]
    return y


def chunked_steps(x, dt, A, B, C, chunk_len, cu_seqlens=None):
    """O3: the block decomposition of [M] §3.5, step by step, in fp64.

    Written from the prose of [M] §3.5.1-3.5.2 and "SSD algorithm: chunking and
    state passing": every sequence is cut into chunks of chunk_len tokens (the
    last one may be shorter; [M] §3.5 notes uneven partitions stay exact) and
      Acs[c, h, l]  = sum_{k<=l} dt_{r0+k} A_h        (chunk-local cumsum)
      1. y_diag[i]  = sum_{j<=i} exp(Acs_i - Acs_j) (C_i . B_j) x_j
                      (each chunk from a zero initial state, the dual form)
      2. S_c        = sum_l exp(Acs_end - Acs_l) x_l (outer) B_l
                      (final state of the chunk from a zero initial state)
      3. Hin[0] = 0, Hin[c+1] = exp(Acs_end(c)) Hin[c] + S_c
                      (true state entering each chunk; last one = final state)
      4. y_off[i]   = exp(Acs_i) (Hin[c] . C_i)
      y = y_diag + y_off.
    Chunks are numbered in packed order over all sequences.  Returns a dict with
    chunk table (seq, start, len), acs (K,H,Q) [entries past len repeat the
    last one], states (K,H,P,N), hin (K,H,P,N), y_diag, y_off, y (Ttot,H,P)
    and final_state (S,H,P,N).
    """
    x = _f64(x)
    H, P = x.shape[-2:]
    if x.ndim == 4 and cu_seqlens is None:
        cu_seqlens = np.arange(x.shape[0] + 1, dtype=np.int64) * x.shape[1]
    Ttot = int(np.prod(x.shape[:-2]))
    x = x.reshape(Ttot, H, P)
    G, N = B.shape[-2:]
    B = _f64(B).reshape(Ttot, G, N)
    C = _f64(C).reshape(Ttot, G, N)
    ell = _f64(dt).reshape(Ttot, H) * _f64(A).reshape(1, H)
    if cu_seqlens is None:
        cu_seqlens = [0, Ttot]
    cu = [int(v) for v in cu_seqlens]
    S = len(cu) - 1
    Q = int(chunk_len)
    table = []
    for s in range(S):
        for t0 in range(cu[s], cu[s + 1], Q):
            table.append((s, t0, min(Q, cu[s + 1] - t0)))
    K = len(table)
    gidx = (np.arange(H) * G) // H
    acs = np.zeros((K, H, Q))
    states = np.zeros((K, H, P, N))
    hin = np.zeros((K, H, P, N))
    y_diag = np.zeros((Ttot, H, P))
    y_off = np.zeros((Ttot, H, P))
    final = np.zeros((S, H, P, N))
    state = {}
    for k, (s, t0, L) in enumerate(table):
        sl = slice(t0, t0 + L)
        cs = np.cumsum(ell[sl], axis=0)  # (L, H)
        acs[k, :, :L] = cs.T
        acs[k, :, L:] = cs[-1][:, None]
        Bc = B[sl][:, gidx, :]  # (L, H, N)
        Cc = C[sl][:, gidx, :]
        Xc = x[sl]  # (L, H, P)
        # step 1: diagonal block, dual (quadratic) form
        seg = cs[:, None, :] - cs[None, :, :]  # (i, j, H)
        causal = np.tril(np.ones((L, L), dtype=bool))[:, :, None]
        Lmask = np.where(causal, np.exp(np.where(causal, seg, 0.0)), 0.0)
        Gm = np.einsum("ihn,jhn->ijh", Cc, Bc)
        y_diag[sl] = np.einsum("ijh,jhp->ihp", Lmask * Gm, Xc)
        # step 2: chunk state from a zero initial state
        w = np.exp(cs[-1][None, :] - cs)  # (L, H)
        states[k] = np.einsum("lh,lhp,lhn->hpn", w, Xc, Bc)
        # step 3: state passing
        h_in = state.get(s, np.zeros((H, P, N)))
        hin[k] = h_in
        state[s] = np.exp(cs[-1])[:, None, None] * h_in + states[k]
        # step 4: state -> output
        y_off[sl] = np.exp(cs)[:, :, None] * np.einsum("hpn,lhn->lhp", h_in, Cc)
    for s in range(S):
        if s in state:
            final[s] = state[s]
    return dict(table=np.array(table, dtype=np.int64).reshape(-1, 3), acs=acs,
                states=states, hin=hin, y_diag=y_diag, y_off=y_off,
                y=y_diag + y_off, final_state=final)


def rel_l2_per_slice(got, ref, slice_axes):
    """Relative L2 error ||got - ref|| / ||ref|| per slice.

    slice_axes: axes that index the slices (e.g. the head axis); the norm runs
    over all other axes.  Returns the array of per-slice errors (a slice whose
    reference is all zero reports the absolute norm of got instead).
    """
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    red = tuple(i for i in range(ref.ndim) if i not in slice_axes)
    num = np.sqrt(np.sum((got - ref) ** 2, axis=red))
    den = np.sqrt(np.sum(ref ** 2, axis=red))
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), num)
