"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Every check here uses a formulation other than the oracle's own recurrence:
brute-force dual form, closed forms of special cases, the linear-attention
cumsum form, the printed 1-SS matrix, structural invariants (rank, causality,
linearity) and decomposition invariances.  A plausible mistake in the oracle (a
dropped term, a wrong sign, an index off by one, a transposed operand, a wrong
head-to-group map) fails at least one of them.

Pages: [T] "Transformers是SSMs：通过结构化状态空间对偶性的广义模型和高效算法(一)"
(nxbn.cn); [M] "LLM(十一)——Mamba" (mztchaoqun.com.cn).
"""
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_case(rng, T, H, P, N, G, dt_lo=1e-3, dt_hi=1e-1):
    x = rng.standard_normal((T, H, P))
    B = rng.standard_normal((T, G, N))
    C = rng.standard_normal((T, G, N))
    dt = np.exp(rng.uniform(math.log(dt_lo), math.log(dt_hi), size=(T, H)))
    A = -np.exp(rng.uniform(0.0, math.log(16.0), size=H))
    return x, dt, A, B, C


def relerr(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


# --------------------------------------------------------------------------
# O1 (recurrence) against O2 (brute-force dual form), [T] §2.4, §3.1 eq. (3)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("T,H,P,N,G", [(1, 1, 1, 1, 1), (7, 2, 3, 4, 1), (40, 4, 5, 6, 2),
                                       (64, 3, 8, 16, 3), (97, 6, 4, 3, 2)])
def test_recurrence_matches_quadratic_form(T, H, P, N, G):
    rng = np.random.default_rng(T * 131 + H)
    x, dt, A, B, C = rand_case(rng, T, H, P, N, G, dt_lo=1e-2, dt_hi=1.0)
    y1, _ = oracle.recurrence(x, dt, A, B, C)
    y2 = oracle.quadratic(x, dt, A, B, C)
    assert relerr(y1, y2) < 1e-12


def test_one_ss_matrix_golden():
    """Probe O1 (N=1, B=C=1) with unit vectors: the 1-SS matrix of [T] §3.2.2."""
    with open(os.path.join(GOLDEN, "one_ss_matrix_T4.txt")) as f:
        rows = [list(map(float, ln.split())) for ln in f if ln.strip() and not ln.startswith("#")]
    a = np.array(rows[0])
    Mref = np.array(rows[1:])
    T = len(a)
    dt = (-np.log(a)).reshape(T, 1)
    A = np.array([1.0]) * -1.0  # a_t = exp(dt_t * A) = exp(ln a_t)
    B = np.ones((T, 1, 1))
    C = np.ones((T, 1, 1))
    M = np.zeros((T, T))
    for i in range(T):
        x = np.zeros((T, 1, 1))
        x[i, 0, 0] = 1.0
        y, _ = oracle.recurrence(x, dt, A, B, C)
        M[:, i] = y[:, 0, 0]
    np.testing.assert_allclose(M, Mref, rtol=1e-14, atol=0)


# --------------------------------------------------------------------------
# Closed forms of special cases
# --------------------------------------------------------------------------
def test_a_one_is_causal_linear_attention():
    """a == 1 (A = 0): causal linear attention, [T] §4.2 / [M] §3.3.2:
    Y = Q . cumsum(K^T V) with (Q, K, V) = (C, B, X), computed as a running sum
    of outer products (the linear form, not the recurrence's decay loop)."""
    rng = np.random.default_rng(5)
    T, H, P, N = 50, 2, 3, 4
    x, dt, _, B, C = rand_case(rng, T, H, P, N, 1)
    A = np.zeros(H)
    y, fs = oracle.recurrence(x, dt, A, B, C)
    KV = np.cumsum(np.einsum("tn,thp->thpn", B[:, 0], x), axis=0)  # (T,H,P,N)
    yref = np.einsum("thpn,tn->thp", KV, C[:, 0])
    assert relerr(y, yref) < 1e-13
    assert relerr(fs[0], KV[-1]) < 1e-13


def test_a_one_unit_vectors_is_prefix_sum():
    """a == 1 and B = C = e_1: y_t = sum_{s<=t} x_s exactly ([M] §3.1.3 with L
    the all-ones lower triangle)."""
    rng = np.random.default_rng(6)
    T, H, P, N = 33, 2, 5, 7
    x = rng.integers(-8, 9, size=(T, H, P)).astype(np.float64)
    B = np.zeros((T, 1, N)); B[:, 0, 0] = 1.0
    C = B.copy()
    dt = np.ones((T, H))
    y, _ = oracle.recurrence(x, dt, np.zeros(H), B, C)
    np.testing.assert_array_equal(y, np.cumsum(x, axis=0))


def test_a_zero_is_diagonal():
    """a == 0 (dt*A = -1e4 underflows exp to 0): L = I, so y_t = (C_t.B_t) x_t
    and the final state is x_{T-1} (outer) B_{T-1} ([T] §3.1 eq. (3): any zero
    factor in a_j...a_{i+1} removes the term)."""
    rng = np.random.default_rng(7)
    T, H, P, N = 20, 3, 4, 5
    x, _, _, B, C = rand_case(rng, T, H, P, N, 1)
    dt = np.full((T, H), 1e4)
    A = -np.ones(H)
    y, fs = oracle.recurrence(x, dt, A, B, C)
    cb = np.einsum("tn,tn->t", C[:, 0], B[:, 0])
    np.testing.assert_allclose(y, cb[:, None, None] * x, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(fs[0], np.einsum("hp,n->hpn", x[-1], B[-1, 0]), rtol=1e-15)


def test_retnet_gamma_closed_form():
    """a == gamma constant, N = 1, B = C = 1, x = 1: the RetNet decay mask of
    [T] §4.3 (structured masked attention instances) gives
    y_t = sum_{s<=t} gamma^{t-s} = (1 - gamma^{t+1}) / (1 - gamma)."""
    T = 300
    for gamma in (0.5, 0.9, 0.999):
        dt = np.ones((T, 1))
        A = np.array([math.log(gamma)])
        y, _ = oracle.recurrence(np.ones((T, 1, 1)), dt, A, np.ones((T, 1, 1)), np.ones((T, 1, 1)))
        t = np.arange(T)
        ref = (1.0 - gamma ** (t + 1)) / (1.0 - gamma)
        np.testing.assert_allclose(y[:, 0, 0], ref, rtol=1e-12)


# --------------------------------------------------------------------------
# Structure and invariants
# --------------------------------------------------------------------------
def test_semiseparable_rank_and_causality():
    """The materialised M (probed column by column) is lower triangular and
    every block below the diagonal has rank <= N ([T] §3.2 Def. 3.1, Lemma
    3.3); generically the rank is exactly N."""
    rng = np.random.default_rng(8)
    T, N = 48, 3
    x0, dt, A, B, C = rand_case(rng, T, 1, 1, N, 1, dt_lo=1e-2, dt_hi=0.3)
    M = np.zeros((T, T))
    for i in range(T):
        x = np.zeros((T, 1, 1)); x[i] = 1.0
        y, _ = oracle.recurrence(x, dt, A, B, C)
        M[:, i] = y[:, 0, 0]
    assert np.all(M[np.triu_indices(T, 1)] == 0.0)
    for k in (8, 20, 33):
        s = np.linalg.svd(M[k:, :k], compute_uv=False)
        assert s[N] <= 1e-12 * s[0]
        assert s[N - 1] > 1e-8 * s[0]


def test_first_decay_of_sequence_is_unused():
    """a_0 of every sequence multiplies the zero initial state: changing dt at
    the first token changes nothing ([T] §3.1: h_0 = B_0 x_0; §3.2.2)."""
    rng = np.random.default_rng(9)
    x, dt, A, B, C = rand_case(rng, 30, 2, 3, 4, 1)
    y1, f1 = oracle.recurrence(x, dt, A, B, C)
    dt2 = dt.copy(); dt2[0] *= 37.0
    y2, f2 = oracle.recurrence(x, dt2, A, B, C)
    np.testing.assert_array_equal(y1, y2)
    np.testing.assert_array_equal(f1, f2)
    dt3 = dt.copy(); dt3[1] *= 37.0  # a_1 does matter
    y3, _ = oracle.recurrence(x, dt3, A, B, C)
    assert not np.array_equal(y1, y3)


def test_linearity_and_causality():
    rng = np.random.default_rng(10)
    x1, dt, A, B, C = rand_case(rng, 40, 2, 3, 4, 1)
    x2 = rng.standard_normal(x1.shape)
    y1, _ = oracle.recurrence(x1, dt, A, B, C)
    y2, _ = oracle.recurrence(x2, dt, A, B, C)
    y12, _ = oracle.recurrence(2.5 * x1 - 0.75 * x2, dt, A, B, C)
    assert relerr(y12, 2.5 * y1 - 0.75 * y2) < 1e-13
    xp = x1.copy(); xp[17] += 1.0
    yp, _ = oracle.recurrence(xp, dt, A, B, C)
    np.testing.assert_array_equal(yp[:17], y1[:17])
    assert not np.array_equal(yp[17:], y1[17:])


def test_split_and_resume():
    """Running [0,T1) and then [T1,T) from its final state equals one run
    (state passing between segments, [M] §3.7 context parallel / §3.5.2)."""
    rng = np.random.default_rng(11)
    x, dt, A, B, C = rand_case(rng, 70, 3, 4, 5, 1)
    y, f = oracle.recurrence(x, dt, A, B, C)
    T1 = 29
    ya, fa = oracle.recurrence(x[:T1], dt[:T1], A, B[:T1], C[:T1])
    yb, fb = oracle.recurrence(x[T1:], dt[T1:], A, B[T1:], C[T1:], init_state=fa)
    assert relerr(np.concatenate([ya, yb]), y) < 1e-13
    assert relerr(fb, f) < 1e-13


def test_skip_term_alone():
    """D passes the input straight to the output ([M] §1.2): with B = 0 no input
    reaches the state, so y = D_h x exactly, on the raw x also when the input
    enters the state as dt x."""
    rng = np.random.default_rng(12)
    x, dt, A, B, C = rand_case(rng, 40, 3, 4, 5, 1)
    B = np.zeros_like(B)
    Dh = rng.standard_normal(3)
    for xdt in (False, True):
        y, f = oracle.recurrence(x, dt, A, B, C, D=Dh, x_times_dt=xdt)
        np.testing.assert_array_equal(y, Dh[None, :, None] * x)
        assert np.all(f == 0)


def test_x_times_dt_is_weighted_prefix_sum():
    """With the input entering as dt x, a == 1 (A = 0) and B = C = e_1:
    y_t = sum_{s<=t} dt_s x_s (a weighted prefix sum), and the final state's
    (p, 0) entries are its last row."""
    rng = np.random.default_rng(13)
    T, H, P, N = 45, 2, 3, 4
    x = rng.standard_normal((T, H, P))
    dt = rng.uniform(0.01, 2.0, size=(T, H))
    B = np.zeros((T, 1, N)); B[:, 0, 0] = 1.0
    C = B.copy()
    y, f = oracle.recurrence(x, dt, np.zeros(H), B, C, x_times_dt=True)
    ref = np.cumsum(dt[:, :, None] * x, axis=0)
    assert relerr(y, ref) < 1e-13
    assert relerr(f[0, :, :, 0], ref[-1]) < 1e-13
    assert np.all(f[0, :, :, 1:] == 0)


def test_varlen_equals_separate_runs():
    """Packed sequences with cu_seqlens restart from a zero state ([M] §3.7.3)
    and equal independent runs, bit for bit; an empty sequence has a zero
    final state."""
    rng = np.random.default_rng(12)
    lens = [5, 0, 17, 1, 9]
    T = sum(lens)
    x, dt, A, B, C = rand_case(rng, T, 2, 3, 4, 2)
    cu = np.concatenate([[0], np.cumsum(lens)])
    y, f = oracle.recurrence(x, dt, A, B, C, cu_seqlens=cu)
    for s in range(len(lens)):
        sl = slice(cu[s], cu[s + 1])
        if lens[s] == 0:
            assert np.all(f[s] == 0)
            continue
        ys, fs = oracle.recurrence(x[sl], dt[sl], A, B[sl], C[sl])
        np.testing.assert_array_equal(y[sl], ys)
        np.testing.assert_array_equal(f[s], fs[0])


def test_group_mapping():
    """G = H with B, C replicated per head equals G = 1; with G = 2 and H = 4,
    heads 0,1 read group 0 and heads 2,3 read group 1 (contiguous blocks)."""
    rng = np.random.default_rng(13)
    x, dt, A, B, C = rand_case(rng, 25, 4, 3, 5, 1)
    y1, f1 = oracle.recurrence(x, dt, A, B, C)
    yH, fH = oracle.recurrence(x, dt, A, np.repeat(B, 4, axis=1), np.repeat(C, 4, axis=1))
    np.testing.assert_array_equal(y1, yH)
    np.testing.assert_array_equal(f1, fH)
    B2 = np.concatenate([B, rng.standard_normal(B.shape)], axis=1)
    C2 = np.concatenate([C, rng.standard_normal(C.shape)], axis=1)
    y2, _ = oracle.recurrence(x, dt, A, B2, C2)
    np.testing.assert_array_equal(y2[:, :2], y1[:, :2])
    assert not np.allclose(y2[:, 2:], y1[:, 2:])


def test_batched_layout_is_packed_sequences():
    rng = np.random.default_rng(14)
    b, T, H, P, N = 3, 11, 2, 3, 4
    x = rng.standard_normal((b, T, H, P)); B = rng.standard_normal((b, T, 1, N))
    C = rng.standard_normal((b, T, 1, N))
    dt = np.exp(rng.uniform(-5, -1, size=(b, T, H))); A = -np.exp(rng.uniform(0, 2, size=H))
    y, f = oracle.recurrence(x, dt, A, B, C)
    assert y.shape == (b, T, H, P) and f.shape == (b, H, P, N)
    for i in range(b):
        yi, fi = oracle.recurrence(x[i], dt[i], A, B[i], C[i])
        np.testing.assert_array_equal(y[i], yi)
        np.testing.assert_array_equal(f[i], fi[0])


# --------------------------------------------------------------------------
# O3 (four-step chunked reference) against O1, each step on its own meaning
# --------------------------------------------------------------------------
@pytest.mark.parametrize("Q,lens", [(8, [64]), (16, [50]), (64, [64]), (32, [7, 40, 0, 33])])
def test_chunked_steps_against_recurrence(Q, lens):
    rng = np.random.default_rng(Q + len(lens))
    T = sum(lens)
    x, dt, A, B, C = rand_case(rng, T, 4, 3, 5, 2, dt_lo=1e-2, dt_hi=0.5)
    cu = np.concatenate([[0], np.cumsum(lens)])
    r = oracle.chunked_steps(x, dt, A, B, C, Q, cu_seqlens=cu)
    y, f = oracle.recurrence(x, dt, A, B, C, cu_seqlens=cu)
    assert relerr(r["y"], y) < 1e-12
    assert relerr(r["final_state"], f) < 1e-12
    a = np.exp(dt * A[None, :])
    for k, (s, t0, L) in enumerate(r["table"]):
        # the cumsum's last entry is the log of the chunk's total decay
        np.testing.assert_allclose(np.exp(r["acs"][k, :, L - 1]), np.prod(a[t0:t0 + L], axis=0),
                                   rtol=1e-12)
        # chunk state = final state of the chunk run alone from zero
        _, fk = oracle.recurrence(x[t0:t0 + L], dt[t0:t0 + L], A, B[t0:t0 + L], C[t0:t0 + L])
        assert relerr(r["states"][k], fk[0]) < 1e-12
        # passed state = final state of the sequence prefix before the chunk
        if t0 == cu[s]:
            assert np.all(r["hin"][k] == 0)
        else:
            _, fp = oracle.recurrence(x[cu[s]:t0], dt[cu[s]:t0], A, B[cu[s]:t0], C[cu[s]:t0])
            assert relerr(r["hin"][k], fp[0]) < 1e-12


def test_rel_l2_metric():
    ref = np.ones((4, 3, 2))
    got = ref.copy()
    got[:, 1, :] *= 1.01
    e = oracle.rel_l2_per_slice(got, ref, slice_axes=(1,))
    np.testing.assert_allclose(e, [0.0, 0.01, 0.0], atol=1e-15)


# --------------------------------------------------------------------------
# O4 (backward) against finite differences of O1 and closed forms
# --------------------------------------------------------------------------
@pytest.mark.parametrize("D_on,xdt", [(False, False), (True, False), (False, True), (True, True)])
def test_backward_matches_finite_differences(D_on, xdt):
    """Every gradient of L = sum(dy . y) + sum(dfinal . h_last) against central
    differences of the forward recurrence (two packed sequences, two groups, an
    initial state): an independent check of the adjoint recurrence."""
    rng = np.random.default_rng(21 + 2 * D_on + xdt)
    T, H, P, N, G = 12, 4, 3, 2, 2
    x, dt, A, B, C = rand_case(rng, T, H, P, N, G, dt_lo=0.05, dt_hi=0.8)
    cu = np.array([0, 7, 12])
    h0 = rng.standard_normal((2, H, P, N))
    dy = rng.standard_normal((T, H, P))
    dfin = rng.standard_normal((2, H, P, N))
    D = rng.standard_normal(H) if D_on else None

    def loss(x_, dt_, A_, B_, C_, h0_, D_):
        y, f = oracle.recurrence(x_, dt_, A_, B_, C_, cu_seqlens=cu, init_state=h0_, D=D_, x_times_dt=xdt)
        return float(np.sum(dy * y) + np.sum(dfin * f))

    g = oracle.backward(x, dt, A, B, C, dy, cu_seqlens=cu, init_state=h0, dfinal=dfin, D=D, x_times_dt=xdt)
    args = [x, dt, A, B, C, h0, D]
    names = ["dx", "ddt", "dA", "dB", "dC", "dinit", "dD"]
    eps = 1e-6
    for k, name in enumerate(names):
        if args[k] is None:
            continue
        fd = np.zeros_like(args[k])
        for idx in np.ndindex(args[k].shape):
            up = [a.copy() if a is not None else None for a in args]
            dn = [a.copy() if a is not None else None for a in args]
            up[k][idx] += eps
            dn[k][idx] -= eps
            fd[idx] = (loss(*up) - loss(*dn)) / (2 * eps)
        np.testing.assert_allclose(g[name], fd, rtol=1e-6, atol=1e-8, err_msg=name)


def test_backward_a_one_prefix_sum():
    """a == 1 and B = C = e_1: y = cumsum(x), so dx is the reverse cumulative sum
    of dy, exactly; the first-token decay of a sequence gets no gradient."""
    rng = np.random.default_rng(22)
    T, H, P, N = 30, 2, 3, 4
    x = rng.integers(-4, 5, size=(T, H, P)).astype(np.float64)
    dy = rng.integers(-4, 5, size=(T, H, P)).astype(np.float64)
    B = np.zeros((T, 1, N)); B[:, 0, 0] = 1.0
    g = oracle.backward(x, np.ones((T, H)), np.zeros(H), B, B.copy(), dy)
    np.testing.assert_array_equal(g["dx"], np.cumsum(dy[::-1], axis=0)[::-1])
    assert np.all(g["ddt"][0] == 0)


def test_backward_a_zero_is_diagonal():
    """a == 0 (dt A = -1e4): y_t = (C_t . B_t) x_t, so dx_t = (C_t . B_t) dy_t,
    dC_t = sum_h (dy_t . x_t) B_t, dB_t = sum_h (dy_t . x_t) C_t, d(dt) = 0."""
    rng = np.random.default_rng(23)
    T, H, P, N = 20, 3, 4, 5
    x, _, _, B, C = rand_case(rng, T, H, P, N, 1)
    dy = rng.standard_normal((T, H, P))
    g = oracle.backward(x, np.full((T, H), 1e4), -np.ones(H), B, C, dy)
    cb = np.einsum("tgn,tgn->t", B, C)
    s = np.einsum("thp,thp->t", dy, x)
    assert relerr(g["dx"], cb[:, None, None] * dy) < 1e-14
    assert relerr(g["dC"], s[:, None, None] * B) < 1e-14
    assert relerr(g["dB"], s[:, None, None] * C) < 1e-14
    assert np.all(g["ddt"] == 0)


# --------------------------------------------------------------------------
# O5 (selective scan with a diagonal transition, the comparator), [M] §3.1.1-
# 3.1.2 and §2.1.2-2.1.3
# --------------------------------------------------------------------------
def scan_case(rng, nb, T, D, N):
    x = rng.standard_normal((nb, T, D))
    delta = np.exp(rng.uniform(math.log(1e-3), math.log(1e-1), size=(nb, T, D)))
    A = -np.exp(rng.uniform(0.0, math.log(16.0), size=(D, N)))
    B = rng.standard_normal((nb, T, N))
    C = rng.standard_normal((nb, T, N))
    return x, delta, A, B, C


def test_selective_scan_scalar_diagonal_is_ssd():
    """With every diagonal entry of a channel's A equal to its head's A_h and
    Delta the head's step size, the diagonal SSM is SSD ([M] §3.1.2) with the
    dt-scaled input: the two oracles agree (O1 is pinned on its own above)."""
    rng = np.random.default_rng(50)
    nb, T, H, P, N = 2, 37, 3, 4, 5
    x, dt, A, B, C = rand_case(rng, nb * T, H, P, N, 1)
    x = x.reshape(nb, T, H, P)
    dt = dt.reshape(nb, T, H)
    B = B.reshape(nb, T, 1, N)
    C = C.reshape(nb, T, 1, N)
    y_ssd, fs_ssd = oracle.recurrence(x, dt, A, B, C, x_times_dt=True)
    delta = np.repeat(dt[..., None], P, axis=-1).reshape(nb, T, H * P)
    Ad = np.repeat(A[:, None], P * N).reshape(H * P, N)
    y, fs = oracle.selective_scan(x.reshape(nb, T, H * P), delta, Ad, B[:, :, 0], C[:, :, 0])
    assert relerr(y, y_ssd.reshape(nb, T, H * P)) < 1e-13
    assert relerr(fs, fs_ssd.reshape(nb, H * P, N)) < 1e-13


def test_selective_scan_a_zero_is_prefix_sum():
    """A = 0 (no decay): h_t = sum_{s<=t} Delta_s x_s B_s, so y_t = C_t . that
    (a closed form by cumulative sums)."""
    rng = np.random.default_rng(51)
    x, delta, A, B, C = scan_case(rng, 2, 30, 3, 4)
    A = np.zeros_like(A)
    y, fs = oracle.selective_scan(x, delta, A, B, C)
    h = np.cumsum((delta * x)[..., None] * B[:, :, None, :], axis=1)  # (b, T, D, N)
    assert relerr(y, np.einsum("btn,btdn->btd", C, h)) < 1e-13
    assert relerr(fs, h[:, -1]) < 1e-13


def test_selective_scan_brute_force_per_state():
    """Brute force by explicit products: y_t[d] = sum_n C_t[n] sum_{s<=t}
    (prod_{s<r<=t} exp(Delta_r[d] A[d,n])) Delta_s[d] B_s[n] x_s[d].  Distinct
    decays per state entry make a wrong n index or a shared decay fail."""
    rng = np.random.default_rng(52)
    nb, T, D, N = 1, 9, 2, 3
    x, delta, A, B, C = scan_case(rng, nb, T, D, N)
    y, _ = oracle.selective_scan(x, delta, A, B, C)
    ref = np.zeros((nb, T, D))
    for b in range(nb):
        for d in range(D):
            for t in range(T):
                acc = 0.0
                for n in range(N):
                    for s in range(t + 1):
                        w = 1.0
                        for r in range(s + 1, t + 1):
                            w *= math.exp(delta[b, r, d] * A[d, n])
                        acc += C[b, t, n] * w * delta[b, s, d] * B[b, s, n] * x[b, s, d]
                ref[b, t, d] = acc
    assert relerr(y, ref) < 1e-13


# --------------------------------------------------------------------------
# O6 (output normalised by the denominator term M 1), [T]/[M] "Incorporating
# a Normalization (Denominator) Term"
# --------------------------------------------------------------------------
def positive_case(rng, T, H, P, N, G):
    """Inputs with a positive feature map on B and C (the pages' condition for
    positive denominators)."""
    x, dt, A, B, C = rand_case(rng, T, H, P, N, G)
    return x, dt, A, np.abs(B) + 0.05, np.abs(C) + 0.05


def test_normalized_ones_input_is_one():
    """X = 1: every output is M 1 / M 1 = 1."""
    rng = np.random.default_rng(60)
    x, dt, A, B, C = positive_case(rng, 50, 3, 4, 5, 1)
    y, _, d = oracle.normalized(np.ones_like(x), dt, A, B, C)
    assert np.max(np.abs(y - 1.0)) < 1e-13
    assert np.all(d > 0)


def test_normalized_brute_force_denominator():
    """The denominator against explicit sums: d_t = sum_{j<=t} (prod_{j<r<=t}
    a_r) C_t . B_j, and y_t = (sum_j (...) x_j) / d_t, by loops."""
    rng = np.random.default_rng(61)
    T, H, P, N = 8, 2, 3, 4
    x, dt, A, B, C = positive_case(rng, T, H, P, N, 1)
    y, _, d = oracle.normalized(x, dt, A, B, C)
    for h in range(H):
        for t in range(T):
            num = np.zeros(P)
            den = 0.0
            for j in range(t + 1):
                w = 1.0
                for r in range(j + 1, t + 1):
                    w *= math.exp(dt[r, h] * A[h])
                cb = float(np.dot(C[t, 0], B[j, 0]))
                num += w * cb * x[j, h]
                den += w * cb
            assert abs(d[t, h] - den) <= 1e-12 * abs(den)
            assert np.max(np.abs(y[t, h] - num / den)) <= 1e-12 * max(1.0, np.max(np.abs(num / den)))


def test_normalized_scale_invariance_and_no_decay_limit():
    """Scaling B (or C) by a positive constant leaves the normalised output
    unchanged; with decays that kill all history (a -> 0) M is diagonal and
    the output is x itself; the skip term is added after the division."""
    rng = np.random.default_rng(62)
    x, dt, A, B, C = positive_case(rng, 40, 2, 3, 4, 1)
    y, _, _ = oracle.normalized(x, dt, A, B, C)
    y2, _, _ = oracle.normalized(x, dt, A, 3.0 * B, 0.5 * C)
    assert relerr(y2, y) < 1e-13
    y0, _, _ = oracle.normalized(x, dt, np.full_like(A, -1e7), B, C)  # dt*A <= -1e4
    assert relerr(y0, x) < 1e-13
    D = np.array([0.5, -2.0])
    yd, _, _ = oracle.normalized(x, dt, A, B, C, D=D)
    assert relerr(yd, y + D[None, :, None] * x) < 1e-13
